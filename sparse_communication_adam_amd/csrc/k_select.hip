// k_select.hip - per-layer top-k of the mask statistic for gfx950.
//
// The mask for step t+1 keeps, in every layer, the k largest statistics with
// ties going to the lower position (per-layer top-k from first-moment
// statistics: gist.science Technical Summary s.2, Partitioned Mask
// Synchronization; the tie rule is the reading this library adopts).  That is
// the top k of the 62-bit composite (key, ~position), found by radix
// selection:
//
//  1. The dense pass histograms the first 11-bit key digit (bits 30..20) per
//     layer.  k_select_first walks the row from the top and picks the bucket
//     holding the k-th element.  If the whole bucket is needed the layer is
//     done; otherwise the bucket's elements are "candidates".
//  2. k_filter reads every key once: keys above the bucket become mask bits
//     (one wave ballot per 64-element word, written as whole words) and the
//     bucket's elements are appended, as (key, layer position) records, to
//     the layer's candidate region (wave-aggregated atomics; record order is
//     irrelevant because the composite order is total).
//  3. Up to five refinement passes over the candidate records only: key bits
//     19..10, key bits 9..0, then, only if the exact threshold key T is tied
//     beyond what is needed, position bits 30..20, 19..10, 9..0 from the
//     smallest position upward.  Each pass is a histogram kernel (LDS row per
//     virtual block, one layer per virtual block) and a per-layer select.
//  4. k_cand_mark sets the bits of the selected candidates with 64-bit atomic
//     ORs on the words the filter already wrote.
//
// Histogram rows are left zeroed by every select kernel, so a row is clean
// for the next pass.
#include "scape_device.h"

namespace scape {

constexpr uint32_t kNone = 0xFFFFFFFFu;

// Generic per-layer bucket search over `nbins` bins of `h`.  Scan order is
// from the top bin down when `descending`, else from bin 0 up.  Returns (via
// LDS) the bucket where the running count first reaches `need`, the count
// before it and the bucket's own count; zeroes the row afterwards.
__device__ void find_bucket(uint32_t* h, int nbins, bool descending, uint32_t need, uint32_t* s_bucket,
                            uint32_t* s_before, uint32_t* s_count, uint32_t* scan_scratch) {
    const int per = nbins / kBlock;  // 8 or 4
    uint32_t c[8];
    uint32_t sum = 0;
    for (int e = 0; e < per; ++e) {
        const int o = threadIdx.x * per + e;
        const int b = descending ? nbins - 1 - o : o;
        c[e] = h[b];
        sum += c[e];
    }
    if (threadIdx.x == 0) *s_bucket = kNone;
    uint32_t before = block_exclusive_scan(sum, scan_scratch, nullptr);
    if (need > 0 && before < need && before + sum >= need) {
        uint32_t cum = before;
        for (int e = 0; e < per; ++e) {
            if (cum + c[e] >= need) {
                const int o = threadIdx.x * per + e;
                *s_bucket = (uint32_t)(descending ? nbins - 1 - o : o);
                *s_before = cum;
                *s_count = c[e];
                break;
            }
            cum += c[e];
        }
    }
    for (int e = 0; e < per; ++e) {
        const int o = threadIdx.x * per + e;
        h[descending ? nbins - 1 - o : o] = 0;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kBlock) void k_select_first(int32_t layer0, const LayerDesc* __restrict__ layers,
                                                         uint32_t* __restrict__ hist, SelState* __restrict__ st) {
    __shared__ uint32_t scratch[kWaves];
    __shared__ uint32_t s_bucket, s_before, s_count;
    const int l = layer0 + blockIdx.x;
    const uint32_t k = layers[l].k;
    find_bucket(hist + (size_t)l * kHistBins, kDigit1Bins, true, k, &s_bucket, &s_before, &s_count, scratch);
    if (threadIdx.x == 0) {
        SelState S{};
        S.J = 0xFFFFFFFFu;
        if (k == 0 || s_bucket == kNone) {
            S.none = 1;
            S.phase = kPhaseDone;
        } else {
            const uint32_t need = k - s_before;
            S.d1 = s_bucket;
            S.kprefix = s_bucket;
            S.need = need;
            if (need == s_count) {  // the whole bucket is kept: key >= d1 << 20
                S.all_bucket = 1;
                S.phase = kPhaseDone;
                S.T = s_bucket << (31 - kDigit1Bits);
            } else {
                S.phase = kPhaseKey2;
                S.cand_count = s_count;
            }
        }
        st[l] = S;
    }
}

hipError_t launch_select_first(hipStream_t s, int32_t layer0, int32_t n_layers, const LayerDesc* layers,
                               uint32_t* hist, SelState* st) {
    if (n_layers <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_select_first, dim3(n_layers), dim3(kBlock), 0, s, layer0, layers, hist, st);
    return hipGetLastError();
}

// Offsets of the layers' candidate regions and of their virtual blocks
// (kCandChunk records each); clears the append counters.  One workgroup of
// 1024 threads, each owning a contiguous run of layers.
__global__ __launch_bounds__(1024) void k_cand_scan(int32_t layer0, int32_t n_layers, uint32_t cand_cap,
                                                    SelState* __restrict__ st, uint32_t* __restrict__ cand_fill,
                                                    uint32_t* __restrict__ totals) {
    __shared__ uint32_t sc[1024], sv[1024];
    const int per = (n_layers + 1023) / 1024;
    const int a = threadIdx.x * per;
    const int b = min(a + per, n_layers);
    uint32_t c = 0, v = 0;
    for (int i = a; i < b; ++i) {
        const uint32_t n = st[layer0 + i].cand_count;
        c += n;
        v += (n + kCandChunk - 1) / kCandChunk;
    }
    sc[threadIdx.x] = c;
    sv[threadIdx.x] = v;
    __syncthreads();
    // Hillis-Steele inclusive scan over 1024 entries
    for (int d = 1; d < 1024; d <<= 1) {
        uint32_t tc = 0, tv = 0;
        if (threadIdx.x >= (unsigned)d) {
            tc = sc[threadIdx.x - d];
            tv = sv[threadIdx.x - d];
        }
        __syncthreads();
        sc[threadIdx.x] += tc;
        sv[threadIdx.x] += tv;
        __syncthreads();
    }
    uint32_t oc = sc[threadIdx.x] - c, ov = sv[threadIdx.x] - v;
    for (int i = a; i < b; ++i) {
        SelState* S = &st[layer0 + i];
        uint32_t n = S->cand_count;
        // Counts come from the same keys the filter reads, so the regions fit
        // the buffer (at most one record per element); clamp anyway so that no
        // record is ever written or read past it.
        if (oc >= cand_cap) n = 0;
        else if (n > cand_cap - oc) n = cand_cap - oc;
        S->cand_count = n;
        S->cand_off = oc;
        S->vblk_off = ov;
        cand_fill[layer0 + i] = 0;
        oc += n;
        ov += (n + kCandChunk - 1) / kCandChunk;
    }
    if (threadIdx.x == 1023) {
        totals[0] = sc[1023];
        totals[1] = sv[1023];
    }
}

hipError_t launch_cand_scan(hipStream_t s, int32_t layer0, int32_t n_layers, uint32_t cand_cap, SelState* st,
                            uint32_t* cand_fill, uint32_t* totals) {
    if (n_layers <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_cand_scan, dim3(1), dim3(1024), 0, s, layer0, n_layers, cand_cap, st, cand_fill, totals);
    return hipGetLastError();
}

// Candidate records are staged in LDS and copied out in bulk: one global
// atomic per flush (normally one per tile) reserves the slots, instead of one
// per word - per-word atomics on a single per-layer counter serialize.
constexpr int kFilterWords = 8;                                 // words per wave per trip
constexpr int kFilterTrip = kWaves * kFilterWords * 64;        // elements per workgroup trip
constexpr int kStage = 2 * kFilterTrip;                         // LDS records (32 KB)

__device__ __forceinline__ void filter_flush(uint32_t* s_n, uint32_t* s_base, const uint64_t* s_rec,
                                             uint32_t* cand_fill, int layer, const SelState& S,
                                             uint64_t* __restrict__ cand) {
    __syncthreads();
    const uint32_t n = *s_n;
    if (n) {
        if (threadIdx.x == 0) *s_base = atomicAdd(&cand_fill[layer], n);
        __syncthreads();
        const uint32_t base = *s_base;
        for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
            const uint32_t slot = base + i;
            if (slot < S.cand_count) cand[(size_t)S.cand_off + slot] = s_rec[i];
        }
        __syncthreads();
        if (threadIdx.x == 0) *s_n = 0;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kBlock) void k_filter(const TileDesc* __restrict__ tiles,
                                                   const LayerDesc* __restrict__ layers,
                                                   const SelState* __restrict__ st, const uint32_t* __restrict__ key,
                                                   uint64_t* __restrict__ bits, uint32_t* __restrict__ cand_fill,
                                                   uint64_t* __restrict__ cand) {
    __shared__ uint64_t s_rec[kStage];
    __shared__ uint32_t s_n, s_base;
    const TileDesc t = tiles[blockIdx.x];
    const LayerDesc L = layers[t.layer];
    const SelState S = st[t.layer];
    const uint32_t lend = L.off + L.n;
    const uint32_t lane = lane_id();
    const uint32_t wave = threadIdx.x / 64;
    const uint32_t d1 = S.d1;
    const bool none = S.none != 0;
    const bool whole = S.all_bucket != 0;
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    // workgroup-uniform trips so that every thread reaches the barriers
    for (uint32_t wb = t.w0; wb < t.w1; wb += kWaves * kFilterWords) {
        const uint32_t w0 = wb + wave * kFilterWords;
        uint32_t kv[kFilterWords];
#pragma unroll
        for (int e = 0; e < kFilterWords; ++e) {
            const uint32_t jj = (w0 + e) * 64u + lane;
            kv[e] = (w0 + e < t.w1 && jj < lend) ? key[jj] : 0u;
        }
        uint64_t mine = 0;
#pragma unroll
        for (int e = 0; e < kFilterWords; ++e) {
            const uint32_t jj = (w0 + e) * 64u + lane;
            const bool inl = (w0 + e < t.w1) && jj < lend && !none;
            const uint32_t d = kv[e] >> (31 - kDigit1Bits);
            const bool sel = inl && (d > d1 || (whole && d == d1));
            const bool cnd = inl && !whole && d == d1;
            const uint64_t word = __ballot(sel);
            if (lane == (uint32_t)e) mine = word;
            const uint64_t cb = __ballot(cnd);
            if (cb) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&s_n, (uint32_t)__popcll(cb));
                base = __shfl(base, 0, 64);
                if (cnd) s_rec[base + lanes_below(cb)] = ((uint64_t)kv[e] << 32) | (uint64_t)(jj - L.off);
            }
        }
        if (lane < (uint32_t)kFilterWords && w0 + lane < t.w1) bits[w0 + lane] = mine;
        __syncthreads();
        if (s_n > (uint32_t)(kStage - kFilterTrip)) filter_flush(&s_n, &s_base, s_rec, cand_fill, t.layer, S, cand);
    }
    filter_flush(&s_n, &s_base, s_rec, cand_fill, t.layer, S, cand);
}

hipError_t launch_filter(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                         const SelState* st, const uint32_t* key, uint64_t* bits, uint32_t* cand_fill,
                         uint64_t* cand) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_filter, dim3(n_tiles), dim3(kBlock), 0, s, tiles, layers, st, key, bits, cand_fill, cand);
    return hipGetLastError();
}

// Layer of virtual candidate block v: the last layer l in [layer0, layer0+n)
// with st[l].vblk_off <= v (offsets are non-decreasing; empty layers share
// the next layer's offset, and the search skips them because their range is
// empty).
__device__ int layer_of_vblock(const SelState* st, int32_t layer0, int32_t n_layers, uint32_t v) {
    int lo = 0, hi = n_layers - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (st[layer0 + mid].vblk_off <= v) lo = mid;
        else hi = mid - 1;
    }
    return layer0 + lo;
}

__device__ __forceinline__ int phase_bins(uint32_t phase) { return phase == kPhasePos1 ? 2048 : 1024; }

__global__ __launch_bounds__(kBlock) void k_cand_hist(uint32_t phase, int32_t layer0, int32_t n_layers,
                                                      const SelState* __restrict__ st,
                                                      const uint32_t* __restrict__ cand_fill,
                                                      const uint32_t* __restrict__ totals,
                                                      const uint64_t* __restrict__ cand,
                                                      uint32_t* __restrict__ hist) {
    __shared__ uint32_t h[2048];
    __shared__ int s_layer;
    const uint32_t nv = totals[1];
    const int nb = phase_bins(phase);
    for (uint32_t v = blockIdx.x; v < nv; v += gridDim.x) {
        if (threadIdx.x == 0) s_layer = layer_of_vblock(st, layer0, n_layers, v);
        __syncthreads();
        const int l = s_layer;
        const SelState S = st[l];
        __syncthreads();
        if (S.phase != phase) continue;  // uniform across the block
        for (int b = threadIdx.x; b < nb; b += kBlock) h[b] = 0;
        __syncthreads();
        const uint32_t chunk = v - S.vblk_off;
        const uint32_t p0 = S.cand_off + chunk * kCandChunk;
        const uint32_t pend = S.cand_off + min(S.cand_count, cand_fill[l]);  // records actually written
        const uint32_t p1 = min(p0 + (uint32_t)kCandChunk, pend);
        for (uint32_t base = p0; base < p1; base += kBlock) {
            const uint32_t p = base + threadIdx.x;
            bool take = false;
            uint32_t digit = 0;
            if (p < p1) {
                const uint64_t rec = cand[p];
                const uint32_t kv = (uint32_t)(rec >> 32), jl = (uint32_t)rec;
                switch (phase) {
                    case kPhaseKey2: take = true; digit = (kv >> 10) & 1023u; break;
                    case kPhaseKey3: take = (kv >> 10) == S.kprefix; digit = kv & 1023u; break;
                    case kPhasePos1: take = kv == S.T; digit = jl >> 20; break;
                    case kPhasePos2: take = kv == S.T && (jl >> 20) == S.jprefix; digit = (jl >> 10) & 1023u; break;
                    default: take = kv == S.T && (jl >> 10) == S.jprefix; digit = jl & 1023u; break;
                }
            }
            hist_add_wave(h, digit, take);
        }
        __syncthreads();
        hist_flush(h, hist + (size_t)l * kHistBins, nb);
        __syncthreads();
    }
}

hipError_t launch_cand_hist(hipStream_t s, uint32_t phase, int32_t layer0, int32_t n_layers, const SelState* st,
                            const uint32_t* cand_fill, const uint32_t* totals, const uint64_t* cand, uint32_t* hist) {
    if (n_layers <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_cand_hist, dim3(1024), dim3(kBlock), 0, s, phase, layer0, n_layers, st, cand_fill, totals,
                       cand, hist);
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_select_next(uint32_t phase, int32_t layer0, uint32_t* __restrict__ hist,
                                                        SelState* __restrict__ st) {
    __shared__ uint32_t scratch[kWaves];
    __shared__ uint32_t s_bucket, s_before, s_count;
    const int l = layer0 + blockIdx.x;
    SelState S = st[l];
    if (S.phase != phase) return;  // uniform
    const bool desc = phase == kPhaseKey2 || phase == kPhaseKey3;
    find_bucket(hist + (size_t)l * kHistBins, phase_bins(phase), desc, S.need, &s_bucket, &s_before, &s_count,
                scratch);
    if (threadIdx.x != 0) return;
    if (s_bucket == kNone) {  // inconsistent counts: select no candidate rather than guess
        S.phase = kPhaseDone;
        S.T = 0xFFFFFFFFu;
        S.J = 0;
        st[l] = S;
        return;
    }
    const uint32_t b = s_bucket;
    const uint32_t need = S.need - s_before;
    const bool exact = need == s_count;  // the whole bucket is kept
    S.need = need;
    switch (phase) {
        case kPhaseKey2:
            S.kprefix = (S.kprefix << 10) | b;
            if (exact) { S.T = S.kprefix << 10; S.J = 0xFFFFFFFFu; S.phase = kPhaseDone; }
            else S.phase = kPhaseKey3;
            break;
        case kPhaseKey3:
            S.T = (S.kprefix << 10) | b;
            if (exact) { S.J = 0xFFFFFFFFu; S.phase = kPhaseDone; }
            else S.phase = kPhasePos1;
            break;
        case kPhasePos1:
            S.jprefix = b;
            if (exact) { S.J = (b << 20) | 0xFFFFFu; S.phase = kPhaseDone; }
            else S.phase = kPhasePos2;
            break;
        case kPhasePos2:
            S.jprefix = (S.jprefix << 10) | b;
            if (exact) { S.J = (S.jprefix << 10) | 1023u; S.phase = kPhaseDone; }
            else S.phase = kPhasePos3;
            break;
        default:
            S.J = (S.jprefix << 10) | b;
            S.phase = kPhaseDone;
            break;
    }
    st[l] = S;
}

hipError_t launch_select_next(hipStream_t s, uint32_t phase, int32_t layer0, int32_t n_layers, uint32_t* hist,
                              SelState* st) {
    if (n_layers <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_select_next, dim3(n_layers), dim3(kBlock), 0, s, phase, layer0, hist, st);
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_cand_mark(int32_t layer0, int32_t n_layers,
                                                      const LayerDesc* __restrict__ layers,
                                                      const SelState* __restrict__ st,
                                                      const uint32_t* __restrict__ cand_fill,
                                                      const uint32_t* __restrict__ totals,
                                                      const uint64_t* __restrict__ cand,
                                                      uint64_t* __restrict__ bits) {
    __shared__ int s_layer;
    const uint32_t nv = totals[1];
    for (uint32_t v = blockIdx.x; v < nv; v += gridDim.x) {
        if (threadIdx.x == 0) s_layer = layer_of_vblock(st, layer0, n_layers, v);
        __syncthreads();
        const int l = s_layer;
        const SelState S = st[l];
        const uint32_t off = layers[l].off;
        const uint32_t n = layers[l].n;
        const uint32_t filled = cand_fill[l];
        __syncthreads();
        if (S.none || S.all_bucket) continue;
        const uint32_t chunk = v - S.vblk_off;
        const uint32_t p0 = S.cand_off + chunk * kCandChunk;
        const uint32_t p1 = min(p0 + (uint32_t)kCandChunk, S.cand_off + min(S.cand_count, filled));
        for (uint32_t p = p0 + threadIdx.x; p < p1; p += kBlock) {
            const uint64_t rec = cand[p];
            const uint32_t kv = (uint32_t)(rec >> 32), jl = (uint32_t)rec;
            if (jl < n && (kv > S.T || (kv == S.T && jl <= S.J))) {
                const uint32_t jj = off + jl;
                atomicOr((unsigned long long*)&bits[jj >> 6], 1ull << (jj & 63u));
            }
        }
    }
}

hipError_t launch_cand_mark(hipStream_t s, int32_t layer0, int32_t n_layers, const LayerDesc* layers,
                            const SelState* st, const uint32_t* cand_fill, const uint32_t* totals,
                            const uint64_t* cand, uint64_t* bits) {
    if (n_layers <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_cand_mark, dim3(1024), dim3(kBlock), 0, s, layer0, n_layers, layers, st, cand_fill, totals,
                       cand, bits);
    return hipGetLastError();
}

}  // namespace scape
