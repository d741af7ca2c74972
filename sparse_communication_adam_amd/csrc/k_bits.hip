// k_bits.hip - 1-bit mask kernels for gfx950: pack, unpack, and the index of
// a mask (ascending positions and the per-word prefix of set bits).
//
// Masks are one bit per element, LSB first in 64-bit words: the packed
// single-bit format of the Memory Optimization paragraph of the gist.science
// Technical Summary, s.2.  On wave64 hardware one word is one wave: a ballot
// over the 64 lanes packs a word, and a masked lane's rank inside its word is
// one mbcnt.
//
// The index is built in three passes over the bits (N/8 bytes each):
// per-workgroup popcounts, one scan of those partial sums, then an emit pass
// that writes block_prefix for every word and the set positions into idx.
#include <mutex>

#include "scape_device.h"

namespace scape {

constexpr int kWordsPerThread = kIndexWordsPerBlock / kBlock;  // 8, thread t owns words t, t+256, ...

__global__ __launch_bounds__(kBlock) void k_index_count(const uint64_t* __restrict__ bits, uint32_t n_words,
                                                        uint32_t* __restrict__ block_sums) {
    __shared__ uint32_t scratch[kWaves];
    const uint32_t wb = blockIdx.x * kIndexWordsPerBlock;
    // unconditional loads at a clamped word (n_words >= 1), so all eight are
    // in flight together; a guarded load becomes a branch and a full wait
    uint64_t w[kWordsPerThread];
#pragma unroll
    for (int e = 0; e < kWordsPerThread; ++e) {
        const uint32_t wi = wb + e * kBlock + threadIdx.x;
        w[e] = bits[wi < n_words ? wi : n_words - 1u];
    }
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < kWordsPerThread; ++e) {
        const uint32_t wi = wb + e * kBlock + threadIdx.x;
        c += wi < n_words ? (uint32_t)__popcll(w[e]) : 0u;
    }
    uint32_t total = 0;
    block_exclusive_scan(c, scratch, &total);
    if (threadIdx.x == 0) block_sums[blockIdx.x] = total;
}

hipError_t launch_index_count(hipStream_t s, const uint64_t* bits, uint32_t n_words, uint32_t* block_sums) {
    const uint32_t nb = (n_words + kIndexWordsPerBlock - 1) / kIndexWordsPerBlock;
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL(k_index_count, dim3(nb), dim3(kBlock), 0, s, bits, n_words, block_sums);
    return hipGetLastError();
}

// Exclusive scan of n_blocks partial sums in place; the total goes to
// block_sums[n_blocks].  One workgroup of 1024 threads, each owning a run.
__global__ __launch_bounds__(1024) void k_index_scan(uint32_t* __restrict__ block_sums, uint32_t n_blocks) {
    __shared__ uint32_t sc[1024];
    const uint32_t per = (n_blocks + 1023) / 1024;
    const uint32_t a = threadIdx.x * per;
    const uint32_t b = min(a + per, n_blocks);
    // the run's sums, eight loads in flight at a time (clamped to the run's
    // last entry, so a thread reads only its own run, and counted only inside it)
    constexpr uint32_t kBatch = 8;
    uint32_t c = 0;
    for (uint32_t i0 = a; i0 < b; i0 += kBatch) {
        uint32_t v[kBatch];
#pragma unroll
        for (uint32_t e = 0; e < kBatch; ++e) v[e] = block_sums[min(i0 + e, b - 1u)];
#pragma unroll
        for (uint32_t e = 0; e < kBatch; ++e) c += i0 + e < b ? v[e] : 0u;
    }
    sc[threadIdx.x] = c;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        uint32_t t = threadIdx.x >= (unsigned)d ? sc[threadIdx.x - d] : 0u;
        __syncthreads();
        sc[threadIdx.x] += t;
        __syncthreads();
    }
    uint32_t off = sc[threadIdx.x] - c;
    for (uint32_t i0 = a; i0 < b; i0 += kBatch) {
        uint32_t v[kBatch];
#pragma unroll
        for (uint32_t e = 0; e < kBatch; ++e) v[e] = block_sums[min(i0 + e, b - 1u)];
#pragma unroll
        for (uint32_t e = 0; e < kBatch; ++e) {
            if (i0 + e < b) {
                block_sums[i0 + e] = off;
                off += v[e];
            }
        }
    }
    if (threadIdx.x == 1023) block_sums[n_blocks] = sc[1023];
}

hipError_t launch_index_scan(hipStream_t s, uint32_t* block_sums, uint32_t n_blocks) {
    hipLaunchKernelGGL(k_index_scan, dim3(1), dim3(1024), 0, s, block_sums, n_blocks);
    return hipGetLastError();
}

// Thread t owns words wb + t + 256e (e < 8): reads and prefix writes are
// contiguous across the workgroup.  The prefix runs in word order through 8
// workgroup scans; each thread then writes the positions of its words' set
// bits (a mask at 1% density has about 0.6 per word, so lanes rarely wait on
// each other; a full mask costs 64 trips, as a wave per word would).
__global__ __launch_bounds__(kBlock) void k_index_emit(const uint64_t* __restrict__ bits, uint32_t n_words,
                                                       const uint32_t* __restrict__ block_offs,
                                                       uint32_t* __restrict__ idx, uint32_t k_cap,
                                                       uint32_t* __restrict__ prefix) {
    __shared__ uint32_t scratch[kWaves];
    const uint32_t wb = blockIdx.x * kIndexWordsPerBlock;
    uint64_t w[kWordsPerThread];
#pragma unroll
    for (int e = 0; e < kWordsPerThread; ++e) {
        const uint32_t wi = wb + e * kBlock + threadIdx.x;
        w[e] = wi < n_words ? bits[wi] : 0ull;
    }
    uint32_t run = block_offs[blockIdx.x];
    uint32_t pre[kWordsPerThread];
#pragma unroll
    for (int e = 0; e < kWordsPerThread; ++e) {
        uint32_t total = 0;
        pre[e] = run + block_exclusive_scan((uint32_t)__popcll(w[e]), scratch, &total);
        run += total;
    }
#pragma unroll
    for (int e = 0; e < kWordsPerThread; ++e) {
        const uint32_t wi = wb + e * kBlock + threadIdx.x;
        if (wi < n_words) prefix[wi] = pre[e];
        uint64_t word = w[e];
        uint32_t r = pre[e];
        while (word) {
            const uint32_t b = (uint32_t)__builtin_ctzll(word);
            if (r < k_cap) idx[r] = wi * 64u + b;
            ++r;
            word &= word - 1;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) prefix[n_words] = block_offs[gridDim.x];
}

hipError_t launch_index_emit(hipStream_t s, const uint64_t* bits, uint32_t n_words, const uint32_t* block_offs,
                             uint32_t* idx, uint32_t k_cap, uint32_t* prefix) {
    const uint32_t nb = (n_words + kIndexWordsPerBlock - 1) / kIndexWordsPerBlock;
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL(k_index_emit, dim3(nb), dim3(kBlock), 0, s, bits, n_words, block_offs, idx, k_cap, prefix);
    return hipGetLastError();
}

// The index of a mask of at most kIndexSmallMaxWords words in two launches
// instead of three, with one word per thread: k_index_count_small counts each
// workgroup's kBlock words, and each workgroup of k_index_emit_small adds up
// the counts of the workgroups before it itself (there are at most kBlock)
// before it emits its words.  For small masks the launches, not the bits,
// take the time.
__global__ __launch_bounds__(kBlock) void k_index_count_small(const uint64_t* __restrict__ bits, uint32_t n_words,
                                                              uint32_t* __restrict__ block_sums) {
    __shared__ uint32_t scratch[kWaves];
    const uint32_t w = blockIdx.x * kBlock + threadIdx.x;
    const uint32_t c = w < n_words ? (uint32_t)__popcll(bits[w]) : 0u;
    uint32_t total = 0;
    block_exclusive_scan(c, scratch, &total);
    if (threadIdx.x == 0) block_sums[blockIdx.x] = total;
}

__global__ __launch_bounds__(kBlock) void k_index_emit_small(const uint64_t* __restrict__ bits, uint32_t n_words,
                                                             const uint32_t* __restrict__ block_sums,
                                                             uint32_t* __restrict__ idx, uint32_t k_cap,
                                                             uint32_t* __restrict__ prefix) {
    __shared__ uint32_t scratch[kWaves];
    __shared__ uint32_t s_off;
    const uint32_t w = blockIdx.x * kBlock + threadIdx.x;
    const uint64_t word = w < n_words ? bits[w] : 0ull;
    const uint32_t bs = threadIdx.x < gridDim.x ? block_sums[threadIdx.x] : 0u;
    uint32_t total = 0;
    const uint32_t before = block_exclusive_scan(bs, scratch, &total);
    if (threadIdx.x == blockIdx.x) s_off = before;
    __syncthreads();
    const uint32_t pre = s_off + block_exclusive_scan((uint32_t)__popcll(word), scratch, nullptr);
    if (w < n_words) prefix[w] = pre;
    if (blockIdx.x == 0 && threadIdx.x == 0) prefix[n_words] = total;
    uint64_t x = word;
    uint32_t r = pre;
    while (x) {
        if (r < k_cap) idx[r] = w * 64u + (uint32_t)__builtin_ctzll(x);
        ++r;
        x &= x - 1;
    }
}

hipError_t launch_index_small(hipStream_t s, const uint64_t* bits, uint32_t n_words, uint32_t* block_sums,
                              uint32_t* idx, uint32_t k_cap, uint32_t* prefix) {
    const uint32_t nb = (n_words + kBlock - 1) / kBlock;
    if (nb == 0 || n_words > kIndexSmallMaxWords) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_index_count_small, dim3(nb), dim3(kBlock), 0, s, bits, n_words, block_sums);
    hipLaunchKernelGGL(k_index_emit_small, dim3(nb), dim3(kBlock), 0, s, bits, n_words, block_sums, idx, k_cap,
                       prefix);
    return hipGetLastError();
}

// The index without a context: the per-workgroup partial sums live in a
// file-scope device array instead of a context workspace, for callers that
// cannot allocate.  Every entry a call reads is written earlier in that call
// (count, then scan), so nothing needs clearing between calls; calls that
// overlap on one GPU share the array and race.
__device__ __align__(256) uint32_t g_index_scratch[kIndexScratchEntries];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t index_scratch(uint32_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // the array's name is a host-side stand-in: its device address on
        // this device (each device holds its own copy) comes from the runtime
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_index_scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// acc |= src over n_words words (the fill-in union of per-worker masks).
__global__ __launch_bounds__(kBlock) void k_or_words(const uint64_t* __restrict__ src, uint64_t* __restrict__ acc,
                                                     uint32_t n_words) {
    for (uint32_t w = blockIdx.x * kBlock + threadIdx.x; w < n_words; w += gridDim.x * kBlock) acc[w] |= src[w];
}

hipError_t launch_or_words(hipStream_t s, const uint64_t* src, uint64_t* acc, uint32_t n_words) {
    if (n_words == 0) return hipSuccess;
    uint32_t blocks = (n_words + kBlock - 1) / kBlock;
    if (blocks > 16384u) blocks = 16384u;
    hipLaunchKernelGGL(k_or_words, dim3(blocks), dim3(kBlock), 0, s, src, acc, n_words);
    return hipGetLastError();
}

// Pack and unpack: a lane takes 16 consecutive elements, so a wave covers a
// 1024-element chunk (16 words) per trip.  The 16 predicate bytes are one
// 16-byte load (or store) when `pred` is 16-byte aligned and the 16 elements
// are inside n; otherwise byte by byte.  Element j is bit j & 63 of word
// j >> 6, so lane l holds bits 16 (l % 4) .. 16 (l % 4) + 15 of word l / 4 of
// its chunk, and lanes 4q .. 4q + 3 together form that word.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint64_t kChunk = 1024;  // elements per wave per trip

// bit b of the result: byte b of x is nonzero (b < 4)
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    const uint32_t t = ((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x;  // top bit of each byte: byte != 0
    return ((t >> 7) & 1u) | ((t >> 14) & 2u) | ((t >> 21) & 4u) | ((t >> 28) & 8u);
}

// bytes 0..3 of the result: bits 0..3 of x (each 0 or 1)
__device__ __forceinline__ uint32_t spread_nibble(uint32_t x) {
    return (x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21);
}

__global__ __launch_bounds__(kBlock) void k_pack(const uint8_t* __restrict__ pred, uint64_t n, uint64_t n_words,
                                                 uint64_t* __restrict__ bits, bool vec) {
    const uint32_t lane = lane_id();
    const uint64_t waves = (uint64_t)gridDim.x * kWaves;
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
    for (uint64_t c = (uint64_t)blockIdx.x * kWaves + threadIdx.x / 64; c < n_chunks; c += waves) {
        const uint64_t j0 = c * kChunk + lane * 16u;
        uint32_t m16 = 0;
        if (vec && j0 + 16u <= n) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(pred + j0);
            m16 = nonzero_bytes(v.x) | (nonzero_bytes(v.y) << 4) | (nonzero_bytes(v.z) << 8) |
                  (nonzero_bytes(v.w) << 12);
        } else {
            for (uint32_t e = 0; e < 16u; ++e)
                if (j0 + e < n && pred[j0 + e] != 0) m16 |= 1u << e;
        }
        const uint32_t m1 = __shfl_down(m16, 1), m2 = __shfl_down(m16, 2), m3 = __shfl_down(m16, 3);
        const uint64_t w = c * (kChunk / 64u) + lane / 4u;
        if ((lane & 3u) == 0 && w < n_words)
            bits[w] = (uint64_t)m16 | ((uint64_t)m1 << 16) | ((uint64_t)m2 << 32) | ((uint64_t)m3 << 48);
    }
}

hipError_t launch_pack(hipStream_t s, const uint8_t* pred, int64_t n, uint64_t* bits) {
    if (n <= 0) return hipSuccess;
    const uint64_t nw = ((uint64_t)n + 63) / 64;
    const uint64_t chunks = ((uint64_t)n + kChunk - 1) / kChunk;
    uint64_t blocks = (chunks + kWaves - 1) / kWaves;
    if (blocks > 16384u) blocks = 16384u;
    const bool vec = ((uintptr_t)pred % 16u) == 0;
    hipLaunchKernelGGL(k_pack, dim3((uint32_t)blocks), dim3(kBlock), 0, s, pred, (uint64_t)n, nw, bits, vec);
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_unpack(const uint64_t* __restrict__ bits, uint64_t n,
                                                   uint8_t* __restrict__ pred, bool vec) {
    const uint32_t lane = lane_id();
    const uint64_t waves = (uint64_t)gridDim.x * kWaves;
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
    for (uint64_t c = (uint64_t)blockIdx.x * kWaves + threadIdx.x / 64; c < n_chunks; c += waves) {
        const uint64_t j0 = c * kChunk + lane * 16u;
        if (j0 >= n) continue;
        const uint32_t m16 = (uint32_t)(bits[j0 >> 6] >> (j0 & 63u)) & 0xFFFFu;
        if (vec && j0 + 16u <= n) {
            u32x4 v;
            v.x = spread_nibble(m16);
            v.y = spread_nibble(m16 >> 4);
            v.z = spread_nibble(m16 >> 8);
            v.w = spread_nibble(m16 >> 12);
            *reinterpret_cast<u32x4*>(pred + j0) = v;
        } else {
            for (uint32_t e = 0; e < 16u; ++e)
                if (j0 + e < n) pred[j0 + e] = (uint8_t)((m16 >> e) & 1u);
        }
    }
}

hipError_t launch_unpack(hipStream_t s, const uint64_t* bits, int64_t n, uint8_t* pred) {
    if (n <= 0) return hipSuccess;
    const uint64_t chunks = ((uint64_t)n + kChunk - 1) / kChunk;
    uint64_t blocks = (chunks + kWaves - 1) / kWaves;
    if (blocks > 16384u) blocks = 16384u;
    const bool vec = ((uintptr_t)pred % 16u) == 0;
    hipLaunchKernelGGL(k_unpack, dim3((uint32_t)blocks), dim3(kBlock), 0, s, bits, (uint64_t)n, pred, vec);
    return hipGetLastError();
}

// Plain device copy for measuring the stream-copy rate the step's kernels
// are compared with: one-shot, 16 bytes per thread, non-temporal loads and
// stores, workgroups in the same XCD-aware order as the dense pass.

__global__ __launch_bounds__(kBlock) void k_copy_probe(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                       uint64_t n16) {
    const uint64_t i = (uint64_t)xcd_block(blockIdx.x, gridDim.x) * kBlock + threadIdx.x;
    if (i >= n16) return;
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

hipError_t launch_copy_probe(hipStream_t s, const void* src, void* dst, uint64_t n16) {
    if (n16 == 0) return hipSuccess;
    const uint64_t blocks = (n16 + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(k_copy_probe, dim3((uint32_t)blocks), dim3(kBlock), 0, s, (const u32x4*)src, (u32x4*)dst,
                       n16);
    return hipGetLastError();
}

// Stream probe: a pass of a given traffic shape and nothing else.  A wave
// per 64-element word reads its lanes' chunk of each source (width bytes
// per lane: 2, 4, 8 or 16), all loads issued before any is used, and
// writes to each destination the XOR of every 32-bit part it read,
// repeated to the destination's width.  Non-temporal loads and stores,
// one-shot workgroups in the dense pass's XCD-aware order.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 probe_load(const uint8_t* base, uint32_t width, size_t e) {
    u32x4 v = {0u, 0u, 0u, 0u};
    const uint8_t* p = base + e * width;
    switch (width) {
        case 2: v.x = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p)); break;
        case 4: v.x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); break;
        case 8: {
            const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
            v.x = t.x;
            v.y = t.y;
            break;
        }
        default: v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); break;
    }
    return v;
}

__device__ __forceinline__ void probe_store(uint8_t* base, uint32_t width, size_t e, uint32_t x) {
    uint8_t* p = base + e * width;
    switch (width) {
        case 2: __builtin_nontemporal_store((uint16_t)x, reinterpret_cast<uint16_t*>(p)); break;
        case 4: __builtin_nontemporal_store(x, reinterpret_cast<uint32_t*>(p)); break;
        case 8: __builtin_nontemporal_store(u32x2{x, x}, reinterpret_cast<u32x2*>(p)); break;
        default: __builtin_nontemporal_store(u32x4{x, x, x, x}, reinterpret_cast<u32x4*>(p)); break;
    }
}

__global__ __launch_bounds__(kBlock) void k_stream_probe(StreamProbe a, uint32_t n_words) {
    const uint32_t w = xcd_block(blockIdx.x, gridDim.x) * kWaves + threadIdx.x / 64;
    if (w >= n_words) return;
    const size_t e = (size_t)w * 64 + (threadIdx.x & 63);
    u32x4 v[kStreamProbeMax];
#pragma unroll
    for (int i = 0; i < kStreamProbeMax; ++i)
        if (i < a.n_src) v[i] = probe_load(a.src[i], a.src_width[i], e);
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kStreamProbeMax; ++i)
        if (i < a.n_src) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
#pragma unroll
    for (int i = 0; i < kStreamProbeMax; ++i)
        if (i < a.n_dst) probe_store(a.dst[i], a.dst_width[i], e, x);
}

hipError_t launch_stream_probe(hipStream_t s, const StreamProbe& a, uint32_t n_words) {
    if (n_words == 0) return hipSuccess;
    const uint32_t blocks = (n_words + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_stream_probe, dim3(blocks), dim3(kBlock), 0, s, a, n_words);
    return hipGetLastError();
}

}  // namespace scape
