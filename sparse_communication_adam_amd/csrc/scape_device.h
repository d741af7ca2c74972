// scape_device.h - wave64 helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scape_internal.h"

namespace scape {

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Mask of the active lanes for which `p` holds.  The compiler builtin takes
// the compare result as it is; the HIP wrapper first widens the predicate to
// an integer and compares it again, two more vector instructions per use.
__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// The compiler's lane-write intrinsic (v_writelane_b32), which this clang
// does not expose as a builtin.  Called through the intrinsic rather than
// written as inline assembly, so that the compiler sees the operands and
// inserts the wait states a lane write needs after a vector instruction
// that wrote its scalar source (a comparison's result, for one).
__device__ int scape_writelane_i32(int value, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Lane `lane` (a constant) of v takes the wave-uniform value u.
__device__ __forceinline__ void write_lane(uint32_t& v, uint32_t u, int lane) {
    v = (uint32_t)scape_writelane_i32((int)u, lane, (int)v);
}

// Workgroups are dispatched to the 8 XCDs in turn (workgroup b to XCD b % 8),
// each with its own L2 and translation caches.  xcd_block(b, n) renumbers the
// n workgroups so that each XCD's share is one contiguous run of [0, n), in
// dispatch order.
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t n) {
    const uint32_t q = n / kXcds, r = n % kXcds;
    const uint32_t x = b % kXcds, k = b / kXcds;
    return x * q + (x < r ? x : r) + k;
}

// Sum of x over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Bit pattern of |v| (sign cleared): the mask statistic's integer key.
__device__ __forceinline__ uint32_t magnitude_key(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t t = __shfl_up(x, d, 64);
        if (lane >= (uint32_t)d) x += t;
    }
    return x;
}

// Exclusive scan over a workgroup of kThreads threads.  `scratch` holds
// kThreads / 64 entries of LDS.  Every thread of the block must call it.
template <int kThreads>
__device__ __forceinline__ uint32_t block_exclusive_scan_t(uint32_t v, uint32_t* scratch, uint32_t* total) {
    constexpr int kNW = kThreads / 64;
    const uint32_t lane = lane_id();
    const uint32_t wave = threadIdx.x / 64;
    uint32_t inc = wave_inclusive_scan(v);
    if (lane == 63) scratch[wave] = inc;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
        uint32_t s = scratch[w];
        if ((uint32_t)w < wave) off += s;
        tot += s;
    }
    __syncthreads();
    if (total) *total = tot;
    return off + inc - v;
}

__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
    return block_exclusive_scan_t<kBlock>(v, scratch, total);
}

// Add one count per active lane with `take` set to lds_hist[bin].  When every
// counting lane of the wave hits one bin (heavy ties), a single atomic adds
// the whole wave's count.
__device__ __forceinline__ void hist_add_wave(uint32_t* lds_hist, uint32_t bin, bool take) {
    const uint64_t act = wave_ballot(take);
    if (act == 0) return;
    if (take) {
        // only the counting lanes run here: the first one's bin, and whether
        // every counting lane has it
        const uint32_t bin0 = __builtin_amdgcn_readfirstlane(bin);
        const uint64_t same = wave_ballot(bin == bin0);
        if (same == act) {
            if (lane_id() == (uint32_t)__builtin_ctzll(act)) atomicAdd(&lds_hist[bin0], (uint32_t)__popcll(act));
        } else {
            atomicAdd(&lds_hist[bin], 1u);
        }
    }
}

// Flush a workgroup's LDS histogram row into the global per-layer row
// (`threads` is the workgroup size).
__device__ __forceinline__ void hist_flush(const uint32_t* lds_hist, uint32_t* row, int bins, int threads = kBlock) {
    for (int b = threadIdx.x; b < bins; b += threads) {
        uint32_t c = lds_hist[b];
        if (c) atomicAdd(&row[b], c);
    }
}

}  // namespace scape
