// k_select.hip - per-layer top-k of the mask statistic for gfx950.
//
// The mask for step t+1 keeps, in every layer, the k largest statistics with
// ties going to the lower position (per-layer top-k from first-moment
// statistics: gist.science Technical Summary s.2, Partitioned Mask
// Synchronization; the tie rule is the reading this library adopts).  That is
// the top k of the 62-bit composite (key, ~position), found by radix
// selection: first on the 13-bit digit d = bits 30..18 of the key (buckets of
// 1/32 octave), then on key bits 17..15, 14..6 and 5..0 and, for ties, on the
// position.  The selection reads 16-bit keys (bits 30..15); the full key of a
// candidate still undecided after the first two digits comes from a
// KeySource.
//
//  1. k_sample_hist histograms d over a 1/16 sample of each layer's words
//     (words picked by a hash of their index, so that no row or column
//     structure aligns with the sample; layers of up to kFullSampleWords words
//     are taken whole).  k_estimate turns the sample into a window [lo, hi] of
//     buckets that holds the bucket of the k-th largest key unless the sample
//     is off by more than kZ standard deviations; a wholly sampled layer gets
//     its exact bucket.
//  2. k_filter reads every key once: d > hi becomes a mask bit (one wave
//     ballot per 64-element word, written as whole words, whose popcounts add
//     up to the exact count above the window); lo <= d <= hi becomes a
//     (key, layer position) record.  Records are staged per wave in LDS and
//     stored in the element range of their record segment (a run of tiles of
//     one layer), with one reservation per workgroup on the segment's counter.
//  3. A first record pass histograms d of the records; with the count above
//     the window, k_select_first finds the exact bucket d1 of the k-th key.  If
//     d1 is outside the window (a sampling miss), k_hist_full and
//     k_filter_exact redo that layer from all its keys, so the result is exact
//     in every case.
//  4. Up to six refinement passes over the records: key bits 17..15, 14..6
//     and 5..0, then - only if the threshold key T is tied beyond what is
//     needed - position bits 30..20, 19..10, 9..0 from the smallest position
//     upward.  Each pass marks the records its layer's decided prefix already
//     selects (64-bit atomic ORs on the words the filter wrote), drops those
//     it rules out, and histograms and compacts the undecided rest, so every
//     pass reads only what the previous one left; a per-layer select kernel
//     then fixes the next digit.  A last pass marks what remains selected.
//
// Histogram rows are left zeroed by every select kernel, so a row is clean
// for the next pass.
#include <type_traits>

#include "scape_device.h"

namespace scape {

constexpr uint32_t kNone = 0xFFFFFFFFu;

// Generic per-layer bucket search over `nbins` bins of `h` (global or LDS)
// by a workgroup of kThreads threads.  Scan order is from the top bin down
// when `descending`, else from bin 0 up.  Returns (via LDS) the bucket where
// the running count first reaches `need`, the count before it and the
// bucket's own count; zeroes the row afterwards.  Each thread owns a
// contiguous run of bins in scan order: one pass sums it, a workgroup scan
// places it, and the one thread whose run holds the target walks it again.
template <int kThreads = kBlock>
__device__ void find_bucket(uint32_t* h, int nbins, bool descending, uint32_t need, uint32_t* s_bucket,
                            uint32_t* s_before, uint32_t* s_count, uint32_t* scan_scratch) {
    const int per = (nbins + kThreads - 1) / kThreads;
    const int e0 = (int)threadIdx.x * per, e1 = min(e0 + per, nbins);  // this thread's run (may be empty)
    auto bin = [&](int o) { return descending ? nbins - 1 - o : o; };
    uint32_t sum = 0;
    for (int e = e0; e < e1; ++e) sum += h[bin(e)];
    if (threadIdx.x == 0) *s_bucket = kNone;
    const uint32_t before = block_exclusive_scan_t<kThreads>(sum, scan_scratch, nullptr);
    if (need > 0 && before < need && before + sum >= need) {
        uint32_t cum = before;
        for (int e = e0; e < e1; ++e) {
            const int b = bin(e);
            const uint32_t c = h[b];
            if (cum + c >= need) {
                *s_bucket = (uint32_t)b;
                *s_before = cum;
                *s_count = c;
                break;
            }
            cum += c;
        }
    }
    __syncthreads();
    for (int e = e0; e < e1; ++e) h[bin(e)] = 0;
    __syncthreads();
}

constexpr uint32_t kSampleShift = 4;            // 1 word in 16
constexpr uint32_t kFullSampleWords = 4096;     // layers up to 262144 elements are taken whole
constexpr float kZ = 6.0f;                      // sampling margin in standard deviations

// kModeNoRecords: the layer's records did not fit its record space even for
// the exact threshold bucket; its remaining digits are decided by passes over
// the layer's keys themselves (key_passes, run by the record passes)
// instead of records.
enum SelMode : uint32_t { kModeWindow = 0, kModeFullHist = 2, kModeReclassify = 1, kModeNoRecords = 3 };

__device__ __forceinline__ uint32_t word_hash(uint32_t w) {
    uint32_t h = w * 0x9E3779B1u;
    h ^= h >> 15;
    h *= 0x85EBCA77u;
    h ^= h >> 13;
    return h;
}

// ---------------------------------------------------------------------------
// 1. sample and window

#ifndef SCAPE_SAMPLE_TILES
#define SCAPE_SAMPLE_TILES 16
#endif
constexpr int kSampleTiles = SCAPE_SAMPLE_TILES;  // tiles per workgroup in the sampling pass
constexpr int kSampleBlock = 1024;  // 16 waves share one 32 KB LDS row: 8 waves per SIMD

// In each aligned group of 16 words of a layer, the sampled word is the one at
// offset hash(group) & 15; layers of up to kFullSampleWords words are taken
// whole.  A workgroup takes kSampleTiles consecutive tiles and flushes its
// LDS row when the layer changes.  The work is lane-parallel: eight lanes per
// sampled word, each loading 16 bytes (8 keys), the hash computed in every
// lane.  The sampled words of all of the workgroup's tiles of large layers
// (32 per 512-word tile: 256 lane tasks per tile, four per lane) are loaded
// at once and then histogrammed tile by tile, so a workgroup waits for memory
// once rather than once per tile; wholly sampled layers are read tile by
// tile.  (Measured against a wave per sampled word walking the tiles in turn
// with the hashing on the scalar unit: 113 against 200 us on the 1.75B
// workload.)
constexpr uint32_t kSampleTaskTile = (kTileWords >> kSampleShift) * 8u;  // lane tasks of a large layer's tile
constexpr uint32_t kSampleTaskSlots = kSampleTiles * kSampleTaskTile / kSampleBlock;
static_assert(kSampleTaskTile * kSampleTiles % kSampleBlock == 0 && kSampleBlock % kSampleTaskTile == 0,
              "a tile's tasks are whole lane groups");
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// add the first `kc` of the 8 keys in v to the LDS row
__device__ __forceinline__ void hist_add8(uint32_t* h, const u32x4& v, uint32_t kc) {
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (uint32_t e = 0; e < 8u; ++e)
        if (e < kc) atomicAdd(&h[((q[e >> 1] >> (16u * (e & 1u))) & 0xFFFFu) >> kDigit1FromKey16], 1u);
}

__global__ __launch_bounds__(kSampleBlock) void k_sample_hist(const TileDesc* __restrict__ tiles, uint32_t n_tiles,
                                                         const LayerDesc* __restrict__ layers,
                                                         const uint16_t* __restrict__ key,
                                                         uint32_t* __restrict__ hist,
                                                         uint32_t* __restrict__ sample_words) {
    __shared__ uint32_t h[kDigit1Bins];
    __shared__ uint32_t s_cnt;
    const uint32_t lane = lane_id();
    const uint32_t t0 = blockIdx.x * kSampleTiles;
    const uint32_t nt = min((uint32_t)kSampleTiles, n_tiles - t0);
    for (int b = threadIdx.x; b < kDigit1Bins; b += kSampleBlock) h[b] = 0;
    if (threadIdx.x == 0) s_cnt = 0;
    // gather: task T = slot * kSampleBlock + thread is tile T / kSampleTaskTile,
    // its sampled word (T / 8) % (tile's words / 16), keys 8 (T % 8) .. +7;
    // a lane without a task loads the array's first 16 bytes
    u32x4 kv[kSampleTaskSlots];
    uint32_t kc[kSampleTaskSlots];
#pragma unroll
    for (uint32_t u = 0; u < kSampleTaskSlots; ++u) {
        const uint32_t T = u * kSampleBlock + threadIdx.x;
        const uint32_t i = T / kSampleTaskTile, sw = (T >> 3) % (kSampleTaskTile / 8u), c = T & 7u;
        uint32_t addr = 0;
        kc[u] = 0;
        if (i < nt) {
            const TileDesc t = tiles[t0 + i];
            const LayerDesc L = layers[t.layer];
            const uint32_t lw0 = L.off / 64u, lwords = (L.n + 63u) / 64u, lend = L.off + L.n;
            if (L.k != 0 && lwords > kFullSampleWords) {
                const uint32_t g = ((t.w0 - lw0) >> kSampleShift) + sw;
                const uint32_t g1 = (t.w1 - lw0 + 15u) >> kSampleShift;
                const uint32_t w = lw0 + (g << kSampleShift) + (word_hash(lw0 + (g << kSampleShift)) & 15u);
                if (g < g1 && w < t.w1) {
                    const uint32_t left = lend - w * 64u;  // keys of the word inside the layer (>= 1)
                    kc[u] = left > 8u * c ? min(left - 8u * c, 8u) : 0u;
                    addr = w * 64u + 8u * c;
                }
            }
        }
        kv[u] = *reinterpret_cast<const u32x4*>(key + addr);
    }
    __syncthreads();
    uint32_t nk = 0;  // keys this lane sampled since the last flush
    int cur = -1;
#pragma unroll
    for (uint32_t i = 0; i < (uint32_t)kSampleTiles; ++i) {
        if (i >= nt) break;
        const TileDesc t = tiles[t0 + i];
        const LayerDesc L = layers[t.layer];
        if (t.layer != cur) {  // uniform
            if (cur >= 0) {
                const uint32_t ws = wave_sum(nk);
                if (lane == 0 && ws) atomicAdd(&s_cnt, ws);
                nk = 0;
                __syncthreads();
                hist_flush(h, hist + (size_t)cur * kHistBins, kDigit1Bins, kSampleBlock);
                if (threadIdx.x == 0 && s_cnt) atomicAdd(&sample_words[cur], s_cnt);
                __syncthreads();
                for (int b = threadIdx.x; b < kDigit1Bins; b += kSampleBlock) h[b] = 0;
                if (threadIdx.x == 0) s_cnt = 0;
                __syncthreads();
            }
            cur = t.layer;
        }
        if (L.k == 0) continue;  // nothing to select: no sample
        const uint32_t lwords = (L.n + 63u) / 64u, lend = L.off + L.n;
        if (lwords > kFullSampleWords) {
            const uint32_t u = i * kSampleTaskTile / kSampleBlock;
            if (threadIdx.x / kSampleTaskTile == i % (kSampleBlock / kSampleTaskTile)) {
                hist_add8(h, kv[u], kc[u]);
                nk += kc[u];
            }
        } else {
            // a wholly sampled layer: every word of the tile, eight lanes per word
            for (uint32_t wb = t.w0; wb < t.w1; wb += kSampleBlock / 8u) {
                const uint32_t w = wb + threadIdx.x / 8u, c = threadIdx.x & 7u;
                const uint32_t left = w < t.w1 ? lend - w * 64u : 0u;
                const uint32_t n8 = left > 8u * c ? min(left - 8u * c, 8u) : 0u;
                const u32x4 v = *reinterpret_cast<const u32x4*>(key + (n8 ? w * 64u + 8u * c : 0u));
                hist_add8(h, v, n8);
                nk += n8;
            }
        }
    }
    if (cur >= 0) {
        const uint32_t ws = wave_sum(nk);
        if (lane == 0 && ws) atomicAdd(&s_cnt, ws);
        __syncthreads();
        hist_flush(h, hist + (size_t)cur * kHistBins, kDigit1Bins, kSampleBlock);
        if (threadIdx.x == 0 && s_cnt) atomicAdd(&sample_words[cur], s_cnt);
    }
}

hipError_t launch_sample_hist(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                              const uint16_t* key, uint32_t* hist, uint32_t* sample_count) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_sample_hist, dim3((n_tiles + kSampleTiles - 1) / kSampleTiles), dim3(kSampleBlock), 0, s, tiles,
                       n_tiles, layers, key, hist, sample_count);
    return hipGetLastError();
}

// Window of buckets for each layer from its sample histogram (sample_count
// keys of n).  With C(b) the sampled count at or above bucket b and
// s = n / sample_count, the true count is about s*C(b) with standard
// deviation about s*sqrt(C(b)); hi is the highest bucket whose count could
// reach k and lo the highest bucket whose count surely does.  A layer taken
// whole (s = 1) is exact: lo = hi = the bucket of the k-th key.
__global__ __launch_bounds__(kBlock) void k_estimate(int32_t layer0, const LayerDesc* __restrict__ layers,
                                                     uint32_t* __restrict__ hist,
                                                     const uint32_t* __restrict__ sample_count,
                                                     SelState* __restrict__ st, uint32_t* __restrict__ miss) {
    __shared__ uint32_t suffix[kDigit1Bins];
    __shared__ uint32_t scratch[kWaves];
    if (blockIdx.x == 0 && threadIdx.x == 0) *miss = 0;  // no layer has missed its window yet
    const int l = layer0 + blockIdx.x;
    const LayerDesc L = layers[l];
    uint32_t* row = hist + (size_t)l * kHistBins;
    // per thread a run of bins from the top; suffix[b] = sampled count at or above b
    constexpr int per = kDigit1Bins / kBlock;
    uint32_t sum = 0;
    for (int e = 0; e < per; ++e) sum += row[kDigit1Bins - 1 - (threadIdx.x * per + e)];
    uint32_t run = block_exclusive_scan(sum, scratch, nullptr);
    for (int e = 0; e < per; ++e) {
        const int b = kDigit1Bins - 1 - (threadIdx.x * per + e);
        run += row[b];
        suffix[b] = run;
        row[b] = 0;  // leave the row clean
    }
    __shared__ int s_hi, s_lo;
    if (threadIdx.x == 0) {
        s_hi = -1;
        s_lo = -1;
    }
    __syncthreads();
    const uint32_t m = sample_count[l];
    if (L.k > 0 && m > 0) {
        // both conditions hold on a run of buckets from 0 upward (the counts
        // at-or-above shrink as b grows), so each is "the largest b where it
        // holds"
        const bool exact = m >= L.n;
        const float sc = exact ? 1.0f : (float)L.n / (float)m;
        const float k = (float)L.k;
        int my_hi = -1, my_lo = -1;
        for (int e = 0; e < per; ++e) {
            const int b = kDigit1Bins - 1 - (threadIdx.x * per + e);
            const float C = (float)suffix[b];
            const float est = sc * C, dev = exact ? 0.0f : kZ * sc * sqrtf(C + 1.0f);
            if (est + dev >= k) my_hi = max(my_hi, b);  // the k-th key may lie in b or below
            if (est - dev >= k) my_lo = max(my_lo, b);  // the k-th key surely lies in b or above
        }
        if (my_hi >= 0) atomicMax(&s_hi, my_hi);
        if (my_lo >= 0) atomicMax(&s_lo, my_lo);
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    SelState S{};
    S.n_lo = 1;
    S.n_hi = 0;  // empty window
    if (L.k > 0 && m > 0) {
        S.n_hi = (uint32_t)max(s_hi, 0);
        S.n_lo = (uint32_t)max(s_lo, 0);
    }
    st[l] = S;
}

hipError_t launch_estimate(hipStream_t s, int32_t layer0, int32_t n_layers, const LayerDesc* layers, uint32_t* hist,
                           const uint32_t* sample_count, SelState* st, uint32_t* miss) {
    if (n_layers <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_estimate, dim3(n_layers), dim3(kBlock), 0, s, layer0, layers, hist, sample_count, st, miss);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 2. the pass over every key

// Words per wave per trip of a key pass: each is one 2-byte load per lane,
// and the next trip's loads are in flight while a trip is processed.  The
// hot key filter takes 16 (measured on 1.75G keys: 4 words 1.24 ms, 8 0.91,
// 16 0.82, 24 0.91, 32 0.95: more in flight until the registers cut the
// waves per SIMD; on the GPT-345M shape at keep 1/10, with records in most
// words, 8, 16 and 24 took 287, 276 and 326 us); the other passes keep 8.
constexpr int kFilterWords = 8;
constexpr int kFilterWordsHot = 16;
constexpr int kWaveStage = 256;                 // staged records per wave (2 KB): 8 KB per workgroup

// Full keys of up to kFetch records of layer L (the bits of `sel` say
// which), in place.  All loads are issued unconditionally at safe indices so
// that the gathers overlap: first the mask word, prefix, residual and m of
// each record, then the sparse-buffer entries those select.
constexpr int kFetch = 4;

__device__ __forceinline__ void candidate_keys(const KeySource& ks, const LayerDesc& L, uint64_t* rec,
                                               uint32_t sel) {
    uint32_t jj[kFetch];
#pragma unroll
    for (int u = 0; u < kFetch; ++u) jj[u] = L.off + (((sel >> u) & 1u) ? (uint32_t)rec[u] : 0u);
    uint32_t kk[kFetch];
    // each source in a branch of its own, so that its kFetch loads are issued
    // before any is used (a select inside the loop compiled to one branch and
    // one wait per record)
    if (ks.mtilde) {
        float f[kFetch];
#pragma unroll
        for (int u = 0; u < kFetch; ++u) f[u] = ks.mtilde[jj[u]];
#pragma unroll
        for (int u = 0; u < kFetch; ++u) kk[u] = magnitude_key(f[u]);
    } else if (ks.key32) {
#pragma unroll
        for (int u = 0; u < kFetch; ++u) kk[u] = ks.key32[jj[u]];
    } else {
        // first the mask word, prefix and owner's residual of each record;
        // then one load per record from the array its mask bit selects: the
        // owner's sparse buffer on the current mask, m off it.  m is never
        // read at a masked position, where the update pass, running beside
        // the selection, writes it.
        const float* r = ks.r[L.owner];
        const float* b = ks.b[L.owner];
        uint64_t word[kFetch];
        uint32_t pre[kFetch];
        float rv[kFetch];
#pragma unroll
        for (int u = 0; u < kFetch; ++u) {
            word[u] = ks.cur_bits[jj[u] >> 6];
            pre[u] = ks.cur_prefix[jj[u] >> 6];
            rv[u] = r[(size_t)(jj[u] >> 6) * ks.ws + (jj[u] & 63u)];
        }
        bool on[kFetch];
        const float* src[kFetch];
#pragma unroll
        for (int u = 0; u < kFetch; ++u) {
            const uint32_t bit = jj[u] & 63u;
            const uint32_t rank = pre[u] + (uint32_t)__popcll(word[u] & ((1ull << bit) - 1ull));
            // with no buffer (k_cap == 0) no position counts as masked
            on[u] = ((word[u] >> bit) & 1ull) && rank < ks.k_cap;
            src[u] = on[u] ? b + rank : ks.m + jj[u];
        }
        float val[kFetch];
#pragma unroll
        for (int u = 0; u < kFetch; ++u) val[u] = *src[u];
#pragma unroll
        for (int u = 0; u < kFetch; ++u) {
            const float bm = ks.beta1 * val[u];
            kk[u] = on[u] ? magnitude_key(val[u]) : magnitude_key(bm + ks.c1 * rv[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < kFetch; ++u)
        if ((sel >> u) & 1u) rec[u] = ((uint64_t)kk[u] << 32) | (rec[u] & 0xFFFFFFFFull);
}

// Write n staged records of a wave at slot `first` of segment G.
__device__ __forceinline__ void wave_store(const uint64_t* stage, uint32_t n, uint32_t first, const SegDesc& G,
                                           uint64_t* __restrict__ cand) {
    for (uint32_t i = lane_id(); i < n; i += 64) {
        const uint32_t slot = first + i;
        if (slot < G.size) cand[(size_t)G.base + slot] = stage[i];
    }
}

// The same, with each record's full key fetched first (candidate_keys), so
// that the records carry all 31 key bits.
__device__ __forceinline__ void wave_store_full(const uint64_t* stage, uint32_t n, uint32_t first, const SegDesc& G,
                                                uint64_t* __restrict__ cand, const KeySource& ks, const LayerDesc& L) {
    const uint32_t lane = lane_id();
    for (uint32_t i0 = 0; i0 < n; i0 += 64u * kFetch) {
        uint64_t rec[kFetch];
        uint32_t sel = 0;
#pragma unroll
        for (uint32_t u = 0; u < (uint32_t)kFetch; ++u) {
            const uint32_t i = i0 + u * 64u + lane;
            rec[u] = i < n ? stage[i] : 0ull;
            if (i < n) sel |= 1u << u;
        }
        candidate_keys(ks, L, rec, sel);
#pragma unroll
        for (uint32_t u = 0; u < (uint32_t)kFetch; ++u) {
            const uint32_t i = i0 + u * 64u + lane;
            if (i < n && first + i < G.size) cand[(size_t)G.base + first + i] = rec[u];
        }
    }
}

// Keys of a tile: first digit d >= sel_from -> mask bit; cand_lo <= d <=
// cand_hi -> record, holding the 16 stored key bits (the low 15 bits zero;
// the pass over key bits 17..9 fetches the full key of the records it still
// needs).  With kHist the records' first digits are also counted into the
// layer's histogram row (bins cand_lo..cand_hi), which the threshold-bucket
// search reads next.  Every word of the tile is written.  The waves work
// alone until the end of the tile, where one reservation on the segment's
// counter places all of the workgroup's records (a wave whose staging fills
// up mid-tile reserves on its own), and the count of bits set is added to the
// segment's total.  Must be called by every thread of the workgroup.
// LDS of the key pass: each wave's staged records, and the workgroup's
// record and bit counts.
constexpr int kFilterHistBins = 512;  // LDS bins of the records' first digits (wider windows count in global memory)
template <int kNW>
struct KeyPassLdsT {
    uint64_t rec[kNW][kWaveStage];
    uint32_t hist[kFilterHistBins];
    uint32_t n[kNW], ab[kNW], fl[kNW], base, reserved;
};
using KeyPassLds = KeyPassLdsT<kWaves>;

// With kFullKeys the records are stored with their full keys, from *ks.
// Returns (in every thread) the record slots the workgroup reserved.
template <bool kRecords, bool kHist = false, int kThreads = kBlock, bool kFullKeys = false, int kWords = kFilterWords>
__device__ __forceinline__ uint32_t key_pass(KeyPassLdsT<kThreads / 64>& lds, const TileDesc& t, const LayerDesc& L, const SegDesc& G,
                                         uint32_t sel_from, uint32_t cand_lo, uint32_t cand_hi,
                                         const uint16_t* __restrict__ key, uint64_t* __restrict__ bits,
                                         uint32_t* __restrict__ seg_fill, uint64_t* __restrict__ cand,
                                         uint32_t* __restrict__ seg_above, uint32_t* __restrict__ hist_row = nullptr,
                                         const KeySource* ks = nullptr) {
    constexpr int kNW = kThreads / 64;
    const uint32_t lend = L.off + L.n;
    // histogram bins of the window's first digits: in LDS when they fit
    const uint32_t width = kHist ? cand_hi - cand_lo + 1u : 0u;
    const bool lds_hist = kHist && width <= (uint32_t)kFilterHistBins;
    if (kHist) {
        for (uint32_t b = threadIdx.x; b < (lds_hist ? width : 0u); b += kThreads) lds.hist[b] = 0;
        __syncthreads();
    }
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    uint64_t* stage = lds.rec[wave];
    // the digit tests on the stored 16-bit key (digit = key >> 3): above is
    // key >= k_above; with records the window ends where the bits begin
    // (every caller passes sel_from = cand_hi + 1), so a record is a key >=
    // k_lo that is not above
    const uint32_t k_above = (kRecords ? cand_hi + 1u : sel_from) << kDigit1FromKey16;
    const uint32_t k_lo = cand_lo << kDigit1FromKey16;
    uint32_t n_st = 0;
    uint32_t flushed = 0;     // records this wave reserved and stored mid-tile
    uint32_t above_lane = 0;  // bits set in the mask words this lane wrote
    constexpr uint32_t kStride = kNW * kWords;
    // The next trip's keys are loaded before this trip is processed.  Every
    // load is issued, at a word of the tile (a word past its end loads the
    // tile's last word and is skipped), so the count of loads in flight is
    // the same on every path and the next trip's loads stay in flight while
    // this one is processed.
    uint32_t nxt[kWords];
    auto load_keys = [&](uint32_t w0, uint32_t* kv) {
        if (w0 + kWords <= t.w1) {  // one base address, the words at immediate offsets
            const uint16_t* p = key + (size_t)w0 * 64u + lane;
#pragma unroll
            for (int e = 0; e < kWords; ++e) kv[e] = p[e * 64];
        } else {
#pragma unroll
            for (int e = 0; e < kWords; ++e) kv[e] = key[(size_t)min(w0 + e, t.w1 - 1u) * 64u + lane];
        }
    };
    // One word: its mask word (kept by lane e) and its records.  `left` is
    // the number of its keys inside the layer (64 for every word but a
    // layer's last).
    auto one_word = [&](auto partial, uint32_t w, uint32_t kw, int e, uint32_t left, uint64_t lmask,
                        uint32_t& mine_lo, uint32_t& mine_hi) {
        const uint64_t above = wave_ballot(kw >= k_above);
        const uint64_t word = above & lmask;
        // lane e keeps the word: two lane writes, no per-lane select
        write_lane(mine_lo, (uint32_t)word, e);
        write_lane(mine_hi, (uint32_t)(word >> 32), e);
        if (kRecords) {
            const uint64_t cb = wave_ballot(kw >= k_lo) & ~above & lmask;
            if (cb) {
                if (n_st > (uint32_t)(kWaveStage - 64)) {  // no room for a whole word: flush
                    uint32_t first = 0;
                    if (lane == 0) first = atomicAdd(&seg_fill[t.seg], n_st);
                    if constexpr (kFullKeys)
                        wave_store_full(stage, n_st, __shfl(first, 0, 64), G, cand, *ks, L);
                    else
                        wave_store(stage, n_st, __shfl(first, 0, 64), G, cand);
                    flushed += n_st;
                    n_st = 0;
                }
                const bool rec = (cb >> lane) & 1u;
                if (rec)
                    stage[n_st + lanes_below(cb)] = ((uint64_t)(kw << kKeyShift) << 32) | (uint64_t)(w * 64u + lane - L.off);
                n_st += (uint32_t)__popcll(cb);
                if (kHist) {
                    const uint32_t bin = (kw >> kDigit1FromKey16) - cand_lo;
                    if (lds_hist) hist_add_wave(lds.hist, bin, rec);
                    else if (rec) atomicAdd(&hist_row[cand_lo + bin], 1u);
                }
            }
        }
    };
    load_keys(t.w0 + wave * kWords, nxt);
    for (uint32_t w0 = t.w0 + wave * kWords; w0 < t.w1; w0 += kStride) {
        uint32_t kv[kWords];
#pragma unroll
        for (int e = 0; e < kWords; ++e) kv[e] = nxt[e];
        load_keys(w0 + kStride, nxt);
        uint32_t mine_lo = 0, mine_hi = 0;  // lane e: the mask word of word w0 + e
        if (w0 + kWords <= t.w1 && (w0 + kWords) * 64u <= lend) {
            // every word of the trip is in the tile and wholly in the layer
#pragma unroll
            for (int e = 0; e < kWords; ++e)
                one_word(std::false_type{}, w0 + e, kv[e], e, 64u, ~0ull, mine_lo, mine_hi);
        } else {
#pragma unroll
            for (int e = 0; e < kWords; ++e) {
                const uint32_t w = w0 + e;
                if (w >= t.w1) break;
                const uint32_t left = lend - w * 64u;  // >= 1 for a word of the tile
                one_word(std::true_type{}, w, kv[e], e, left, left >= 64u ? ~0ull : (1ull << left) - 1ull, mine_lo,
                         mine_hi);
            }
        }
        const uint64_t mine = ((uint64_t)mine_hi << 32) | mine_lo;
        if (lane < (uint32_t)kWords && w0 + lane < t.w1) {
            bits[w0 + lane] = mine;
            above_lane += (uint32_t)__popcll(mine);
        }
    }
    const uint32_t n_above = wave_sum(above_lane);
    if (lane == 0) {
        lds.n[wave] = n_st;
        lds.ab[wave] = n_above;
        lds.fl[wave] = flushed;
    }
    __syncthreads();
    if (lds_hist) hist_flush(lds.hist, hist_row + cand_lo, (int)width, kThreads);
    if (threadIdx.x == 0) {
        uint32_t tot = 0, ab = 0, fl = 0;
        for (int q = 0; q < kNW; ++q) {
            tot += lds.n[q];
            ab += lds.ab[q];
            fl += lds.fl[q];
        }
        lds.base = tot ? atomicAdd(&seg_fill[t.seg], tot) : 0u;
        lds.reserved = tot + fl;
        if (ab) atomicAdd(&seg_above[t.seg], ab);
    }
    __syncthreads();
    uint32_t first = lds.base;
    const uint32_t reserved = lds.reserved;
    for (uint32_t q = 0; q < wave; ++q) first += lds.n[q];
    if constexpr (kFullKeys)
        wave_store_full(stage, n_st, first, G, cand, *ks, L);
    else
        wave_store(stage, n_st, first, G, cand);
    return reserved;
}

__global__ __launch_bounds__(kBlock) void k_filter(const TileDesc* __restrict__ tiles,
                                                   const LayerDesc* __restrict__ layers,
                                                   const SegDesc* __restrict__ segs,
                                                   const SelState* __restrict__ st, const uint16_t* __restrict__ key,
                                                   uint64_t* __restrict__ bits, uint32_t* __restrict__ seg_fill,
                                                   uint64_t* __restrict__ cand, uint32_t* __restrict__ seg_above,
                                                   uint32_t* __restrict__ hist) {
    const TileDesc t = tiles[blockIdx.x];
    const LayerDesc L = layers[t.layer];
    const SegDesc G = segs[t.seg];
    const SelState S = st[t.layer];
    const bool win = S.n_lo <= S.n_hi && L.k > 0;
    __shared__ KeyPassLds lds;
    // no window (nothing to select, or an empty sample): no bits, no records
    if (win)
        key_pass<true, true, kBlock, false, kFilterWordsHot>(lds, t, L, G, S.n_hi + 1, S.n_lo, S.n_hi, key, bits,
                                                             seg_fill, cand, seg_above,
                             hist + (size_t)t.layer * kHistBins);
    else  // no window (nothing to select, or an empty sample): no bits, no records
        key_pass<false>(lds, t, L, G, (uint32_t)kDigit1Bins, 1u, 0u, key, bits, seg_fill, cand, seg_above);
}

hipError_t launch_filter(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                         const SegDesc* segs, const SelState* st, const uint16_t* key, uint64_t* bits,
                         uint32_t* seg_fill, uint64_t* cand, uint32_t* seg_above, uint32_t* hist) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_filter, dim3(n_tiles), dim3(kBlock), 0, s, tiles, layers, segs, st, key, bits, seg_fill,
                       cand, seg_above, hist);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 3. threshold bucket

__device__ __forceinline__ void init_found(SelState& S, uint32_t k, uint32_t bucket, uint32_t before,
                                           uint32_t count) {
    const uint32_t need = k - before;
    S.d1 = bucket;
    S.kprefix = bucket;
    S.need = need;
    S.all_bucket = need == count;
    S.J = 0xFFFFFFFFu;
    if (S.all_bucket) {  // the whole bucket is kept: key >= d1 << kDigit1Shift
        S.phase = kPhaseDone;
        S.T = bucket << kDigit1Shift;
    } else {
        S.phase = kPhaseKey2;
    }
}

// first_pass = true: hist holds the records' first digits, and the layer's
// segments hold the exact count above the window.  first_pass = false: only
// layers in kModeFullHist, whose hist row now holds every key.
__global__ __launch_bounds__(kBlock) void k_select_first(int32_t layer0, bool first_pass,
                                                         const LayerDesc* __restrict__ layers,
                                                         const uint32_t* __restrict__ layer_seg0,
                                                         uint32_t* __restrict__ hist, SelState* __restrict__ st,
                                                         const uint32_t* __restrict__ seg_above,
                                                         uint32_t* __restrict__ seg_fill,
                                                         const uint32_t* __restrict__ ovf,
                                                         uint32_t* __restrict__ miss) {
    __shared__ uint32_t scratch[kWaves];
    __shared__ uint32_t s_bucket, s_before, s_count, s_above;
    const int l = layer0 + blockIdx.x;
    const SelState old = st[l];
    if (!first_pass && old.mode != kModeFullHist) return;  // uniform
    const uint32_t k = layers[l].k;
    const uint32_t sg0 = layer_seg0[l], sg1 = layer_seg0[l + 1];
    if (threadIdx.x == 0) s_above = 0;
    __syncthreads();
    if (first_pass) {
        uint32_t part = 0;
        for (uint32_t g = sg0 + threadIdx.x; g < sg1; g += kBlock) part += seg_above[g];
        if (part) atomicAdd(&s_above, part);
    }
    __syncthreads();
    const uint32_t a = s_above;
    const bool win = old.n_lo <= old.n_hi;
    // bucket search over the row, starting from the count above the window
    const uint32_t need = (first_pass && a >= k) ? 0u : k - a;
    find_bucket(hist + (size_t)l * kHistBins, kDigit1Bins, true, need, &s_bucket, &s_before, &s_count, scratch);
    if (threadIdx.x != 0) return;
    SelState S{};
    S.n_lo = old.n_lo;
    S.n_hi = old.n_hi;
    if (k == 0) {
        S.none = 1;
        S.phase = kPhaseDone;
        S.J = 0xFFFFFFFFu;
        S.mode = kModeWindow;
    } else if (first_pass && (!win || a >= k || s_bucket == kNone || ovf[l])) {
        // outside the window (or no window, or more records than the layer's
        // record space holds): count every key of the layer
        S.mode = kModeFullHist;
        S.none = 1;  // provisional; the second pass decides
        S.phase = kPhaseDone;
        for (uint32_t g = sg0; g < sg1; ++g) seg_fill[g] = 0;  // the exact pass makes new records
        atomicOr(miss, 1u);  // the fallback kernels have work
    } else if (s_bucket == kNone) {  // cannot happen with a full row; select nothing rather than guess
        S.none = 1;
        S.phase = kPhaseDone;
        S.mode = kModeReclassify;
    } else {
        init_found(S, k, s_bucket, s_before + a, s_count);
        S.mode = first_pass ? kModeWindow : kModeReclassify;
    }
    st[l] = S;
}

hipError_t launch_select_first(hipStream_t s, int32_t layer0, int32_t n_layers, bool first_pass,
                               const LayerDesc* layers, const uint32_t* layer_seg0, uint32_t* hist, SelState* st,
                               const uint32_t* seg_above, uint32_t* seg_fill, const uint32_t* ovf, uint32_t* miss) {
    if (n_layers <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_select_first, dim3(n_layers), dim3(kBlock), 0, s, layer0, first_pass, layers, layer_seg0,
                       hist, st, seg_above, seg_fill, ovf, miss);
    return hipGetLastError();
}

// The sampling-miss path.  Normally no layer needs it, so both kernels run as
// a small grid that walks the tile table and skips tiles of other layers.
constexpr uint32_t kFallbackGrid = 1024;

// Full first-digit histogram of the layers in kModeFullHist.
__global__ __launch_bounds__(kBlock) void k_hist_full(const TileDesc* __restrict__ tiles, uint32_t n_tiles,
                                                      const LayerDesc* __restrict__ layers,
                                                      const SelState* __restrict__ st,
                                                      const uint16_t* __restrict__ key, uint32_t* __restrict__ hist,
                                                      const uint32_t* __restrict__ miss) {
    __shared__ uint32_t h[kDigit1Bins];
    if (*miss == 0) return;  // no layer missed its window: nothing to count
    const uint32_t lane = lane_id();
    for (uint32_t ti = blockIdx.x; ti < n_tiles; ti += gridDim.x) {
        const TileDesc t = tiles[ti];
        if (st[t.layer].mode != kModeFullHist) continue;  // uniform
        const LayerDesc L = layers[t.layer];
        for (int b = threadIdx.x; b < kDigit1Bins; b += kBlock) h[b] = 0;
        __syncthreads();
        const uint32_t lend = L.off + L.n;
        for (uint32_t w = t.w0 + threadIdx.x / 64; w < t.w1; w += kWaves) {
            const uint32_t jj = w * 64u + lane;
            const bool inl = jj < lend;
            hist_add_wave(h, (inl ? (uint32_t)key[jj] : 0u) >> kDigit1FromKey16, inl);
        }
        __syncthreads();
        hist_flush(h, hist + (size_t)t.layer * kHistBins, kDigit1Bins);
        __syncthreads();
    }
}

hipError_t launch_hist_full(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                            const SelState* st, const uint16_t* key, uint32_t* hist, const uint32_t* miss) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_hist_full, dim3(min(n_tiles, kFallbackGrid)), dim3(kBlock), 0, s, tiles, n_tiles, layers, st,
                       key, hist, miss);
    return hipGetLastError();
}

// Reclassification (bits and records from the exact bucket) of the layers in
// kModeReclassify.
__global__ __launch_bounds__(kBlock) void k_filter_exact(const TileDesc* __restrict__ tiles, uint32_t n_tiles,
                                                         const LayerDesc* __restrict__ layers,
                                                         const SegDesc* __restrict__ segs,
                                                         const SelState* __restrict__ st,
                                                         const uint16_t* __restrict__ key,
                                                         uint64_t* __restrict__ bits, uint32_t* __restrict__ seg_fill,
                                                         uint64_t* __restrict__ cand, uint32_t* __restrict__ seg_above,
                                                         const uint32_t* __restrict__ miss) {
    __shared__ KeyPassLds lds;
    if (*miss == 0) return;  // no layer missed its window: nothing to reclassify
    for (uint32_t ti = blockIdx.x; ti < n_tiles; ti += gridDim.x) {
        const TileDesc t = tiles[ti];
        const SelState S = st[t.layer];
        if (S.mode != kModeReclassify || S.none) continue;  // uniform per workgroup
        const LayerDesc L = layers[t.layer];
        const SegDesc G = segs[t.seg];
        if (S.all_bucket)  // keys in the threshold bucket and above, no records
            key_pass<false>(lds, t, L, G, S.d1, 1, 0, key, bits, seg_fill, cand, seg_above);
        else  // above the bucket: bits; in it: records
            key_pass<true>(lds, t, L, G, S.d1 + 1, S.d1, S.d1, key, bits, seg_fill, cand, seg_above);
        __syncthreads();  // the next tile reuses the LDS staging
    }
}

hipError_t launch_filter_exact(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                               const SegDesc* segs, const SelState* st, const uint16_t* key, uint64_t* bits,
                               uint32_t* seg_fill, uint64_t* cand, uint32_t* seg_above,
                               const uint32_t* miss) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_filter_exact, dim3(min(n_tiles, kFallbackGrid)), dim3(kBlock), 0, s, tiles, n_tiles, layers,
                       segs, st, key, bits, seg_fill, cand, seg_above, miss);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 4. records

// Record blocks: each segment's records are cut into blocks of at most
// kCandChunk; block v holds vb_count[v] records starting at cand[vb[v].p0].
// One workgroup of 1024 threads numbers the blocks of the segments
// [seg0, seg0 + n_segs), each thread owning a contiguous run of segments, and
// writes every block's descriptor and initial count.
// A segment whose fill counter passed its record space (G.size) lost records:
// after the key filter (`second` false; no blocks are made then) its layer is
// flagged in ovf, and k_select_first sends it down the exact path; after the
// exact filter (`second` true) the layer switches to kModeNoRecords (bit 1 of
// *miss tells the record passes to run key_passes).
__global__ __launch_bounds__(1024) void k_cand_scan(uint32_t seg0, uint32_t n_segs,
                                                    const SegDesc* __restrict__ segs,
                                                    const uint32_t* __restrict__ seg_fill,
                                                    VblockDesc* __restrict__ vb, uint32_t* __restrict__ vb_count,
                                                    uint32_t* __restrict__ totals, bool second,
                                                    uint32_t* __restrict__ ovf, SelState* __restrict__ st,
                                                    uint32_t* __restrict__ miss) {
    __shared__ uint32_t sv[1024];
    const uint32_t per = (n_segs + 1023) / 1024;
    const uint32_t a = threadIdx.x * per;
    const uint32_t b = min(a + per, n_segs);
    uint32_t v = 0;
    for (uint32_t i = a; i < b; ++i) {
        const SegDesc G = segs[seg0 + i];
        const uint32_t f = seg_fill[seg0 + i];
        if (f > G.size) {  // records were dropped
            if (second) {
                st[G.layer].mode = kModeNoRecords;
                atomicOr(miss, 2u);
            } else {
                ovf[G.layer] = 1u;
            }
        }
        const uint32_t n = min(f, G.size);
        v += (n + kCandChunk - 1) / kCandChunk;
    }
    if (!second) return;  // after the key filter only the overflow flags are needed
    sv[threadIdx.x] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const uint32_t t = threadIdx.x >= (unsigned)d ? sv[threadIdx.x - d] : 0u;
        __syncthreads();
        sv[threadIdx.x] += t;
        __syncthreads();
    }
    uint32_t ov = sv[threadIdx.x] - v;
    for (uint32_t i = a; i < b; ++i) {
        const SegDesc G = segs[seg0 + i];
        const uint32_t n = min(seg_fill[seg0 + i], G.size);
        for (uint32_t c = 0; c < n; c += kCandChunk, ++ov) {
            vb[ov] = VblockDesc{G.base + c, G.layer};
            vb_count[ov] = min((uint32_t)kCandChunk, n - c);
        }
    }
    if (threadIdx.x == 1023) totals[1] = sv[1023];
}

hipError_t launch_cand_scan(hipStream_t s, uint32_t seg0, uint32_t n_segs, const SegDesc* segs,
                            const uint32_t* seg_fill, VblockDesc* vb, uint32_t* vb_count, uint32_t* totals,
                            bool second, uint32_t* ovf, SelState* st, uint32_t* miss) {
    if (n_segs == 0) return hipSuccess;
    hipLaunchKernelGGL(k_cand_scan, dim3(1), dim3(1024), 0, s, seg0, n_segs, segs, seg_fill, vb, vb_count, totals,
                       second, ovf, st, miss);
    return hipGetLastError();
}

constexpr int kPassBins = 2048;  // LDS histogram of a record pass

// Bins of a refinement digit (the first digit is histogrammed relative to the
// layer's window instead).
__device__ __forceinline__ int phase_bins(uint32_t phase) {
    // bucket searches walk whole kBlock-multiples of bins; the narrow digits
    // use the first 2^bits of 256
    if (phase == kPhaseKey2 || phase == kPhaseKey4) return 256;
    if (phase == kPhaseKey3) return 1 << kKey3Bits;
    return phase == kPhasePos1 ? 2048 : 1024;
}

// One record under the state of its layer: 1 = selected, 2 = undecided (its
// digit goes to the phase's histogram), 0 = not selected.  The records a
// layer still holds are exactly the ones left undecided by its previous
// phase, so each rule only has to split those.  Keys rank descending,
// positions ascending.
__device__ __forceinline__ uint32_t classify(uint32_t phase, const SelState& S, uint32_t kv, uint32_t jl,
                                             uint32_t* digit) {
    switch (phase) {
        case kPhaseKey2: {  // stored bits suffice
            const uint32_t d = kv >> kDigit1Shift;
            *digit = (kv >> kKeyShift) & ((1u << kKey2Bits) - 1u);
            return d > S.d1 ? 1u : (d == S.d1 ? 2u : 0u);
        }
        case kPhaseKey3: {  // classified on the stored bits; the digit of a kept record is taken after its fetch
            const uint32_t p = kv >> kKeyShift;
            *digit = 0;
            return p > S.kprefix ? 1u : (p == S.kprefix ? 2u : 0u);
        }
        case kPhaseKey4: {
            const uint32_t p = kv >> kKey4Bits;
            *digit = kv & ((1u << kKey4Bits) - 1u);
            return p > S.kprefix ? 1u : (p == S.kprefix ? 2u : 0u);
        }
        case kPhasePos1:
            *digit = jl >> 20;
            return kv > S.T ? 1u : (kv == S.T ? 2u : 0u);
        case kPhasePos2: {  // every record left has key T
            const uint32_t p = jl >> 20;
            *digit = (jl >> 10) & 1023u;
            return p < S.jprefix ? 1u : (p == S.jprefix ? 2u : 0u);
        }
        case kPhasePos3: {
            const uint32_t p = jl >> 10;
            *digit = jl & 1023u;
            return p < S.jprefix ? 1u : (p == S.jprefix ? 2u : 0u);
        }
        default:  // done: the final rule
            *digit = 0;
            return (kv > S.T || (kv == S.T && jl <= S.J)) ? 1u : 0u;
    }
}

constexpr int kKeyWordGroups = 4;  // groups of kFetch words per wave and trip in key_pass_words

// One phase over the keys of words [w0, w1) of layer L in kModeNoRecords,
// standing in for a record pass: every element of the layer's exact
// threshold bucket d1 is classified by the same rule a record of it would be
// (classify, plus the key test that the record passes leave to compaction),
// with its full key fetched only where its stored 16 bits equal the
// threshold prefix (elsewhere those 16 bits decide).  An intermediate phase
// adds the undecided elements' digits to the LDS histogram h; the final
// phase (kPhaseDone) marks every element the final rule selects (keys above
// the bucket were set by the exact filter).  Every thread of the workgroup
// (kThreads) must call it.  Each wave loads the keys of kKeyWordGroups *
// kFetch words at once and fetches full keys for kFetch words at a time.
template <int kThreads>
__device__ void key_pass_words(uint32_t phase, uint32_t w0, uint32_t w1, const LayerDesc& L, const SelState& S,
                               const uint16_t* __restrict__ key, const KeySource& ks, uint64_t* __restrict__ bits,
                               uint32_t* h) {
    constexpr uint32_t kW = kThreads / 64;
    constexpr uint32_t kTrip = kKeyWordGroups * kFetch;  // words per wave and trip
    const uint32_t lane = lane_id(), wave = threadIdx.x / 64;
    const bool final_pass = phase == kPhaseDone;
    // top 16 bits of the threshold prefix decided so far
    const uint32_t p16 = phase == kPhaseKey3   ? S.kprefix
                         : phase == kPhaseKey4 ? S.kprefix >> kKey3Bits
                                               : S.T >> kKeyShift;
    const uint32_t lend = L.off + L.n;
    for (uint32_t wb = w0 + wave * kTrip; wb < w1; wb += kW * kTrip) {
        // all of the trip's key loads first (a word past the range or a key
        // past the layer loads the layer's first key and is skipped)
        uint32_t kv16[kTrip];
#pragma unroll
        for (uint32_t u = 0; u < kTrip; ++u) {
            const uint32_t j = (wb + u) * 64u + lane;
            kv16[u] = key[(wb + u < w1 && j < lend) ? j : L.off];
        }
#pragma unroll
        for (uint32_t g = 0; g < kTrip; g += kFetch) {
            uint64_t rec[kFetch];
            bool cand[kFetch];
            uint32_t sel = 0;  // bit u: word g + u needs its full key
#pragma unroll
            for (uint32_t u = 0; u < kFetch; ++u) {
                const uint32_t j = (wb + g + u) * 64u + lane;
                cand[u] = wb + g + u < w1 && j < lend && (kv16[g + u] >> kDigit1FromKey16) == S.d1;
                if (cand[u] && phase != kPhaseKey2 && kv16[g + u] == p16) sel |= 1u << u;
                rec[u] = ((uint64_t)(kv16[g + u] << kKeyShift) << 32) | (uint64_t)(cand[u] ? j - L.off : 0u);
            }
            if (wave_ballot(sel != 0u)) candidate_keys(ks, L, rec, sel);
#pragma unroll
            for (uint32_t u = 0; u < kFetch; ++u) {
                const uint32_t j = (wb + g + u) * 64u + lane;
                const uint32_t kv = (uint32_t)(rec[u] >> 32);
                uint32_t digit = 0;
                uint32_t c = cand[u] ? classify(phase, S, kv, j - L.off, &digit) : 0u;
                // the rules of the later position digits assume the set they
                // split holds only keys equal to T, as a layer's records do by
                // then; here every element of the bucket is seen again
                if ((phase == kPhasePos2 || phase == kPhasePos3) && cand[u] && kv != S.T) c = kv > S.T ? 1u : 0u;
                if (final_pass) {
                    if (c == 1u) atomicOr((unsigned long long*)&bits[j >> 6], 1ull << (j & 63u));
                } else {
                    if (phase == kPhaseKey3) digit = (kv >> kKey4Bits) & ((1u << kKey3Bits) - 1u);
                    hist_add_wave(h, digit, c == 2u);
                }
            }
        }
    }
}

// The key passes of the layers in kModeNoRecords, run by the record pass's
// workgroups after their record blocks, walking the tile table; normally no
// layer needs them (bit 1 of *miss clear).  h is the workgroup's LDS
// histogram, free on entry; every thread must call it.
template <int kThreads>
__device__ void key_passes(uint32_t phase, const TileDesc* __restrict__ tiles, uint32_t n_tiles,
                           const LayerDesc* __restrict__ layers, const SelState* __restrict__ st,
                           const uint16_t* __restrict__ key, const KeySource& ks, uint32_t* __restrict__ hist,
                           uint64_t* __restrict__ bits, uint32_t* h) {
    const bool final_pass = phase == kPhaseDone;
    const int nb = final_pass ? 0 : phase_bins(phase);
    for (uint32_t ti = blockIdx.x; ti < n_tiles; ti += gridDim.x) {
        const TileDesc t = tiles[ti];
        const SelState S = st[t.layer];
        // uniform per workgroup: only this kind of layer, in this phase
        if (S.mode != kModeNoRecords || S.none || S.phase != phase) continue;
        const LayerDesc L = layers[t.layer];
        for (int b = threadIdx.x; b < nb; b += kThreads) h[b] = 0;
        __syncthreads();
        key_pass_words<kThreads>(phase, t.w0, t.w1, L, S, key, ks, bits, h);
        __syncthreads();
        if (!final_pass) hist_flush(h, hist + (size_t)t.layer * kHistBins, nb, kThreads);
        __syncthreads();
    }
}

constexpr int kPassBlock = 512;                          // threads per workgroup of a record pass
constexpr int kPassWaves = kPassBlock / 64;
constexpr int kRecPerThread = kCandChunk / kPassBlock;  // 16 records held in registers per thread

// A layer already done at the passes over key bits 17..15 or 14..6 was
// decided on the stored bits (T a multiple of 2^15, J = all positions), so
// the final rule holds on the filter's partial keys too.
//
// One pass over the record blocks (the records' first digits were counted by
// the key filter).  For each block, by the state of its layer: a layer in
// `phase` has its selected records marked,
// its undecided ones histogrammed and compacted to the front of the block,
// the rest dropped; a layer already done has its selected records marked and
// the block emptied.  Each workgroup takes a contiguous range of blocks and
// flushes its LDS histogram only when the layer changes.
__global__ __launch_bounds__(kPassBlock) void k_cand_pass(uint32_t phase, const VblockDesc* __restrict__ vb,
                                                      uint32_t* __restrict__ vb_count,
                                                      const uint32_t* __restrict__ totals,
                                                      const LayerDesc* __restrict__ layers,
                                                      const SelState* __restrict__ st, KeySource ks,
                                                      uint64_t* __restrict__ cand, uint32_t* __restrict__ hist,
                                                      uint64_t* __restrict__ bits, const TileDesc* __restrict__ tiles,
                                                      uint32_t n_tiles, const uint16_t* __restrict__ key,
                                                      const uint32_t* __restrict__ miss) {
    __shared__ uint32_t h[kPassBins];
    __shared__ uint32_t s_wsum[kPassWaves];
    const uint32_t nv = totals[1];
    const uint32_t per = (nv + gridDim.x - 1) / gridDim.x;
    const uint32_t v0 = blockIdx.x * per, v1 = min(v0 + per, nv);
    const uint32_t lane = lane_id(), wave = threadIdx.x / 64;
    int cur = -1;
    uint32_t* cur_row = nullptr;  // global bins of the LDS row (first bin)
    int cur_nb = 0;               // bins to flush
    for (int b = threadIdx.x; b < kPassBins; b += kPassBlock) h[b] = 0;
    for (uint32_t v = v0; v < v1; ++v) {
        const uint32_t cnt = vb_count[v];
        if (cnt == 0) continue;  // uniform
        const VblockDesc D = vb[v];
        const int l = D.layer;
        const SelState S = st[l];
        if (S.none || S.mode == kModeNoRecords) {  // nothing here, or decided without records
            if (threadIdx.x == 0) vb_count[v] = 0;
            continue;
        }
        const uint32_t cph = S.phase;
        if (cph != phase && cph != kPhaseDone) continue;  // not reached: a layer is in this phase or done
        const bool hist_on = cph != kPhaseDone;
        const int nbl = hist_on ? phase_bins(cph) : 0;
        if (hist_on && l != cur) {
            if (cur >= 0) {
                __syncthreads();
                if (cur_nb) hist_flush(h, cur_row, cur_nb, kPassBlock);
                __syncthreads();
                for (int b = threadIdx.x; b < kPassBins; b += kPassBlock) h[b] = 0;
            }
            cur = l;
            cur_row = hist + (size_t)l * kHistBins;
            cur_nb = nbl;
            __syncthreads();
        }
        const LayerDesc Ld = layers[l];
        const uint32_t off = Ld.off, n = Ld.n;
        // the filter's records carry only the 16 stored key bits: enough for
        // the first two digits and for a layer decided on them; the pass over
        // key bits 14..6 fetches the full key of each record it keeps
        const bool fetch = cph == kPhaseKey3;
        // every record load is unconditional, at a slot clamped to the block's
        // last record (cnt >= 1 here), so the 16 loads are in flight together
        uint64_t rec[kRecPerThread];
#pragma unroll
        for (int i = 0; i < kRecPerThread; ++i) {
            const uint32_t p = threadIdx.x + i * kPassBlock;
            rec[i] = cand[(size_t)D.p0 + (p < cnt ? p : cnt - 1u)];
        }
#pragma unroll
        for (int i = 0; i < kRecPerThread; ++i)
            if (threadIdx.x + i * kPassBlock >= cnt) rec[i] = 0ull;
        uint32_t und = 0;  // bit i: record i undecided
#pragma unroll
        for (int i = 0; i < kRecPerThread; ++i) {
            if ((uint32_t)(i * kPassBlock) + wave * 64u >= cnt) break;  // uniform per wave
            const uint32_t p = threadIdx.x + i * kPassBlock;
            const uint32_t kv = (uint32_t)(rec[i] >> 32), jl = (uint32_t)rec[i];
            uint32_t digit = 0;
            const uint32_t c = p < cnt ? classify(cph, S, kv, jl, &digit) : 0u;
            if (c == 1u && jl < n) {
                const uint32_t jj = off + jl;
                atomicOr((unsigned long long*)&bits[jj >> 6], 1ull << (jj & 63u));
            }
            if (hist_on && !fetch) hist_add_wave(h, digit, c == 2u);
            if (c == 2u) und |= 1u << i;
        }
        if (fetch) {
#pragma unroll
            for (int g = 0; g < kRecPerThread; g += kFetch) {
                const uint32_t sel = (und >> g) & ((1u << kFetch) - 1u);
                if (__ballot(sel != 0u) == 0) continue;  // the wave holds none of these
                candidate_keys(ks, Ld, &rec[g], sel);
            }
#pragma unroll
            for (int i = 0; i < kRecPerThread; ++i) {
                if ((uint32_t)(i * kPassBlock) + wave * 64u >= cnt) break;  // uniform per wave
                const uint32_t digit = ((uint32_t)(rec[i] >> 32) >> kKey4Bits) & ((1u << kKey3Bits) - 1u);
                hist_add_wave(h, digit, (und >> i) & 1u);
            }
        }
        {
            // compaction in place: every record of the block is in registers
            // once the barrier is passed, so the writes cannot clobber a
            // record not yet read
            uint32_t wsum = 0;
#pragma unroll
            for (int i = 0; i < kRecPerThread; ++i) wsum += (uint32_t)__popcll(__ballot((und >> i) & 1u));
            if (lane == 0) s_wsum[wave] = wsum;
            __syncthreads();
            uint32_t base = 0, total = 0;
            for (uint32_t q = 0; q < (uint32_t)kPassWaves; ++q) {
                if (q < wave) base += s_wsum[q];
                total += s_wsum[q];
            }
#pragma unroll
            for (int i = 0; i < kRecPerThread; ++i) {
                const bool u = (und >> i) & 1u;
                const uint64_t bm = __ballot(u);
                if (u) cand[(size_t)D.p0 + base + lanes_below(bm)] = rec[i];
                base += (uint32_t)__popcll(bm);
            }
            if (threadIdx.x == 0) vb_count[v] = total;
        }
        __syncthreads();
    }
    if (cur >= 0) {
        __syncthreads();
        if (cur_nb) hist_flush(h, cur_row, cur_nb, kPassBlock);
    }
    if (*miss & 2u) {  // layers decided without records: the same phase over their keys
        __syncthreads();
        key_passes<kPassBlock>(phase, tiles, n_tiles, layers, st, key, ks, hist, bits, h);
    }
}

hipError_t launch_cand_pass(hipStream_t s, uint32_t phase, const VblockDesc* vb, uint32_t* vb_count,
                            const uint32_t* totals, const LayerDesc* layers, const SelState* st,
                            const KeySource& ks, uint64_t* cand, uint32_t* hist, uint64_t* bits,
                            const TileDesc* tiles, uint32_t n_tiles, const uint16_t* key, const uint32_t* miss) {
    hipLaunchKernelGGL(k_cand_pass, dim3(1024), dim3(kPassBlock), 0, s, phase, vb, vb_count, totals, layers, st, ks, cand,
                       hist, bits, tiles, n_tiles, key, miss);
    return hipGetLastError();
}

// The state of a layer after the bucket search of `phase` found bucket b,
// with `before` undecided keys ahead of it in scan order and `count` in it:
// the next digit to resolve, or the final rule once the bucket is taken
// whole or the last digit is known.
__device__ __forceinline__ void advance(SelState& S, uint32_t phase, uint32_t b, uint32_t before, uint32_t count) {
    const uint32_t need = S.need - before;
    const bool exact = need == count;  // the whole bucket is kept
    S.need = need;
    switch (phase) {
        case kPhaseKey2:
            S.kprefix = (S.kprefix << kKey2Bits) | b;
            if (exact) { S.T = S.kprefix << kKeyShift; S.J = 0xFFFFFFFFu; S.phase = kPhaseDone; }
            else S.phase = kPhaseKey3;
            break;
        case kPhaseKey3:
            S.kprefix = (S.kprefix << kKey3Bits) | b;
            if (exact) { S.T = S.kprefix << kKey4Bits; S.J = 0xFFFFFFFFu; S.phase = kPhaseDone; }
            else S.phase = kPhaseKey4;
            break;
        case kPhaseKey4:
            S.T = (S.kprefix << kKey4Bits) | b;
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
}

__global__ __launch_bounds__(kBlock) void k_select_next(uint32_t phase, int32_t layer0, uint32_t* __restrict__ hist,
                                                        SelState* __restrict__ st) {
    __shared__ uint32_t scratch[kWaves];
    __shared__ uint32_t s_bucket, s_before, s_count;
    const int l = layer0 + blockIdx.x;
    SelState S = st[l];
    if (S.phase != phase) return;  // uniform
    const bool desc = phase == kPhaseKey2 || phase == kPhaseKey3 || phase == kPhaseKey4;
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
    advance(S, phase, s_bucket, s_before, s_count);
    st[l] = S;
}

hipError_t launch_select_next(hipStream_t s, uint32_t phase, int32_t layer0, int32_t n_layers, uint32_t* hist,
                              SelState* st) {
    if (n_layers <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_select_next, dim3(n_layers), dim3(kBlock), 0, s, phase, layer0, hist, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 5. the compact path
//
// Where every layer of a range is small, the passes above cost more in
// launches than in work (a step over one 1024x1024 layer ran some 25 short
// kernels back to back).  The compact path makes the same mask in two
// launches, each tile split over `parts` workgroups:
//  - k_compact_hist histograms the first digit of every key of the range;
//    the workgroup that finishes a layer last (a ticket per layer, drawn
//    after a device-scope fence) finds the layer's exact threshold bucket d1
//    from the full row;
//  - k_compact_filter turns keys above d1 into mask bits and keys in it into
//    records, reserved on one counter per layer in the layer's whole record
//    space; the layer's last workgroup then resolves every remaining digit
//    alone - LDS histogram, bucket search, compaction in place - and marks
//    what the final rule selects.  A layer whose bucket did not fit its
//    record space is resolved the same way from its keys (bit 1 of *miss).
// Each ticket is put back to zero by the workgroup that draws its last
// number.

constexpr int kCompactBlock = 1024;  // threads of the filtering and finishing workgroups
constexpr int kCompactWaves = kCompactBlock / 64;
constexpr int kFinRecs = 8;          // records per thread per chunk in the finishing workgroup

// Tiles of a layer: its words cut every kTileWords from its first word.
__device__ __forceinline__ uint32_t layer_tiles(const LayerDesc& L) {
    return ((L.n + 63u) / 64u + kTileWords - 1u) / kTileWords;
}

// Part p of `parts` of tile t: words [*w0, *w1) (possibly empty).
__device__ __forceinline__ void tile_part(const TileDesc& t, uint32_t parts, uint32_t p, uint32_t* w0,
                                          uint32_t* w1) {
    const uint32_t span = (t.w1 - t.w0 + parts - 1u) / parts;
    *w0 = min(t.w0 + p * span, t.w1);
    *w1 = min(*w0 + span, t.w1);
}

// Draw this workgroup's ticket for `layer` after its writes; true (in every
// thread) for the workgroup that completes the layer's `n` tickets, which
// may then read every other workgroup's writes to global memory.  Each wave
// first waits for its own stores and atomics, so that the one release (the
// ticket, drawn by thread 0 after a write-back of its L2) covers the whole
// workgroup.  In the last workgroup every wave then acquires for itself
// (invalidating the caches it reads through): an invalidation issued by
// another wave is not known to be complete when the barrier lets this one
// load.
template <int kThreads>
__device__ __forceinline__ bool last_of_layer(uint32_t* ticket, int layer, uint32_t n, uint32_t* s_flag) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&ticket[layer], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == n - 1u;
        if (last) ticket[layer] = 0u;  // every other ticket is drawn: reset for the next pass
        *s_flag = last ? 1u : 0u;
    }
    __syncthreads();
    const bool last = *s_flag != 0u;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return last;
}

// The same with a 64-bit ticket word per layer whose low half also sums the
// workgroups' `count`s: the last workgroup gets the layer's total in *total
// (the record counter's final value, without reading it back).
template <int kThreads>
__device__ __forceinline__ bool last_of_layer_sum(unsigned long long* ticket, int layer, uint32_t n, uint32_t count,
                                                  uint32_t* s_flag, uint32_t* s_total, uint32_t* total) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long prev = __hip_atomic_fetch_add(&ticket[layer], (1ull << 32) | count, __ATOMIC_RELEASE,
                                                               __HIP_MEMORY_SCOPE_AGENT);
        const bool last = (uint32_t)(prev >> 32) == n - 1u;
        if (last) ticket[layer] = 0ull;
        *s_flag = last ? 1u : 0u;
        *s_total = (uint32_t)prev + count;
    }
    __syncthreads();
    const bool last = *s_flag != 0u;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *total = *s_total;
    return last;
}

constexpr int kCompactHistBatch = 4;  // 16-byte key loads in flight per thread

__global__ __launch_bounds__(kCompactBlock) void k_compact_hist(const TileDesc* __restrict__ tiles, uint32_t parts,
                                                         const LayerDesc* __restrict__ layers,
                                                         const uint16_t* __restrict__ key,
                                                         uint32_t* __restrict__ hist, SelState* __restrict__ st,
                                                         uint32_t* __restrict__ ticket,
                                                         uint32_t* __restrict__ lrec,
                                                         uint32_t* __restrict__ labove,
                                                         uint32_t* __restrict__ miss) {
    __shared__ __align__(16) uint32_t h[kDigit1Bins];
    __shared__ uint32_t scratch[kCompactWaves];
    __shared__ uint32_t s_flag, s_bucket, s_before, s_count;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *miss = 0;
    const TileDesc t = tiles[blockIdx.x];
    const LayerDesc L = layers[t.layer];
    uint32_t w0, w1;
    tile_part(t, parts, blockIdx.y, &w0, &w1);
    if (L.k > 0) {  // uniform
        for (int b = threadIdx.x; b < kDigit1Bins; b += kCompactBlock) h[b] = 0;
        __syncthreads();
        const uint32_t lend = L.off + L.n;
        // 16-byte chunks (8 keys) of the part, kCompactHistBatch per thread in
        // flight; a chunk past the part or the layer loads the part's first
        const uint32_t nch = (w1 - w0) * 8u;
        for (uint32_t c0 = 0; c0 < nch; c0 += kCompactHistBatch * kCompactBlock) {
            u32x4 v[kCompactHistBatch];
            uint32_t kc[kCompactHistBatch];
#pragma unroll
            for (int i = 0; i < kCompactHistBatch; ++i) {
                const uint32_t c = c0 + i * kCompactBlock + threadIdx.x;
                const uint32_t e = w0 * 64u + 8u * c;
                kc[i] = (c < nch && e < lend) ? min(lend - e, 8u) : 0u;
                v[i] = *reinterpret_cast<const u32x4*>(key + (kc[i] ? e : w0 * 64u));
            }
#pragma unroll
            for (int i = 0; i < kCompactHistBatch; ++i) hist_add8(h, v[i], kc[i]);
        }
        __syncthreads();
        hist_flush(h, hist + (size_t)t.layer * kHistBins, kDigit1Bins, kCompactBlock);
    }
    if (!last_of_layer<kCompactBlock>(ticket, t.layer, layer_tiles(L) * parts, &s_flag)) return;
    // the exact threshold bucket from the layer's full row, searched in LDS
    // (the row is left zeroed)
    {
        u32x4* row = reinterpret_cast<u32x4*>(hist + (size_t)t.layer * kHistBins);
        constexpr int kVec = kDigit1Bins / 4 / kCompactBlock;
        u32x4 v[kVec];
#pragma unroll
        for (int i = 0; i < kVec; ++i) v[i] = row[threadIdx.x + i * kCompactBlock];
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
            reinterpret_cast<u32x4*>(h)[threadIdx.x + i * kCompactBlock] = v[i];
            row[threadIdx.x + i * kCompactBlock] = z;
        }
        __syncthreads();
    }
    find_bucket<kCompactBlock>(h, kDigit1Bins, true, L.k, &s_bucket, &s_before, &s_count, scratch);
    if (threadIdx.x != 0) return;
    SelState S{};
    S.n_lo = 1;
    S.n_hi = 0;
    S.mode = kModeReclassify;
    if (L.k == 0 || s_bucket == kNone) {  // nothing to select (a full row always holds the k-th key)
        S.none = 1;
        S.phase = kPhaseDone;
        S.J = 0xFFFFFFFFu;
    } else {
        init_found(S, L.k, s_bucket, s_before, s_count);
    }
    st[t.layer] = S;
    lrec[t.layer] = 0u;
    labove[t.layer] = 0u;
}

hipError_t launch_compact_hist(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, uint32_t parts,
                               const LayerDesc* layers, const uint16_t* key, uint32_t* hist, SelState* st,
                               uint32_t* ticket, uint32_t* lrec, uint32_t* labove, uint32_t* miss) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_compact_hist, dim3(n_tiles, parts), dim3(kCompactBlock), 0, s, tiles, parts, layers, key, hist, st,
                       ticket, lrec, labove, miss);
    return hipGetLastError();
}

// LDS of the finishing workgroup: its histogram and state, and the records
// once at most kFinLdsRecs remain.  It shares the key pass's LDS, which is
// free by then.
constexpr uint32_t kFinLdsRecs = 3072;
constexpr uint32_t kWaveRecs = 256;  // records one wave finishes faster alone than the workgroup
constexpr int kFinDigitBits = kKey2Bits + kKey3Bits;  // 12: key bits 17..6 in one digit
constexpr int kFinBins = 1 << kFinDigitBits;
static_assert(kFinBins >= kPassBins, "the finishing histogram holds every digit");
struct FinishLds {
    uint64_t rec[kFinLdsRecs];
    alignas(16) uint32_t h[kFinBins];
    uint32_t scratch[kCompactWaves];
    uint32_t wsum[kCompactWaves];
    uint32_t bucket, before, count;
    SelState S;
};
union CompactLds {
    KeyPassLdsT<kCompactWaves> pass;
    FinishLds fin;
};

// The bucket search closing `phase` of layer L, finished by one workgroup:
// the layer's next state in f.S.  With `merged`, the phase of key bits
// 17..15 took bits 17..6 as one 12-bit digit (records with full keys): its
// bucket fixes both digits at once, as the two searches would have.  In a
// layer of at most 2^20 elements every position's bits 30..20 are zero, so
// that digit's search is skipped (its bucket would be 0, never taken whole).
__device__ __forceinline__ void finish_select(FinishLds& f, uint32_t phase, const LayerDesc& L, bool merged) {
    const bool wide = merged && phase == kPhaseKey2;
    const bool desc = phase == kPhaseKey2 || phase == kPhaseKey3 || phase == kPhaseKey4;
    find_bucket<kCompactBlock>(f.h, wide ? kFinBins : phase_bins(phase), desc, f.S.need, &f.bucket, &f.before,
                               &f.count, f.scratch);
    if (threadIdx.x == 0) {
        SelState S = f.S;
        if (f.bucket == kNone) {  // inconsistent counts: select no candidate rather than guess
            S.phase = kPhaseDone;
            S.T = 0xFFFFFFFFu;
            S.J = 0;
        } else if (wide) {
            S.need -= f.before;
            S.kprefix = (S.kprefix << kFinDigitBits) | f.bucket;
            if (S.need == f.count) {  // the whole bucket is kept
                S.T = S.kprefix << kKey4Bits;
                S.J = 0xFFFFFFFFu;
                S.phase = kPhaseDone;
            } else {
                S.phase = kPhaseKey4;
            }
        } else {
            advance(S, phase, f.bucket, f.before, f.count);
        }
        if (S.phase == kPhasePos1 && L.n <= (1u << 20)) {
            S.jprefix = 0;
            S.phase = kPhasePos2;
        }
        f.S = S;
    }
    __syncthreads();
}

// Bucket search by one wave over `nbins` LDS bins (a multiple of 64), in
// the order and with the result of find_bucket; zeroes the bins.  False if
// no bucket reaches `need`.
__device__ __forceinline__ bool wave_find_bucket(uint32_t* h, int nbins, bool descending, uint32_t need,
                                                 uint32_t* bucket, uint32_t* before, uint32_t* count) {
    const uint32_t lane = lane_id();
    const int per = nbins / 64;
    auto bin = [&](int o) { return descending ? nbins - 1 - o : o; };
    uint32_t sum = 0;
    for (int e = 0; e < per; ++e) sum += h[bin((int)lane * per + e)];
    const uint32_t inc = wave_inclusive_scan(sum);
    const bool mine = need > 0 && inc - sum < need && inc >= need;
    uint32_t b = 0, bef = 0, cnt = 0;
    if (mine) {
        uint32_t cum = inc - sum;
        for (int e = 0; e < per; ++e) {
            const uint32_t c = h[bin((int)lane * per + e)];
            if (cum + c >= need) {
                b = (uint32_t)bin((int)lane * per + e);
                bef = cum;
                cnt = c;
                break;
            }
            cum += c;
        }
    }
    for (int e = 0; e < per; ++e) h[bin((int)lane * per + e)] = 0;
    const uint64_t who = wave_ballot(mine);
    if (who == 0) return false;
    const int src = __builtin_ctzll(who);
    *bucket = __shfl(b, src, 64);
    *before = __shfl(bef, src, 64);
    *count = __shfl(cnt, src, 64);
    return true;
}

// The remaining phases of a layer by wave 0 alone, once its `cnt` records
// are in LDS: the same rules, counts and compaction as finish_records, with
// no workgroup barrier between them.
__device__ void finish_wave(FinishLds& f, const LayerDesc& L, uint32_t cnt, uint64_t* __restrict__ bits) {
    const uint32_t lane = lane_id();
    SelState S = f.S;
    for (;;) {
        const uint32_t phase = S.phase;
        const bool final_pass = phase == kPhaseDone;
        uint32_t out = 0;
        for (uint32_t p0 = 0; p0 < cnt; p0 += 64) {
            const uint32_t p = p0 + lane;
            const uint64_t r = p < cnt ? f.rec[p] : 0ull;
            const uint32_t kv = (uint32_t)(r >> 32), jl = (uint32_t)r;
            uint32_t digit = 0;
            uint32_t c = p < cnt ? classify(phase, S, kv, jl, &digit) : 0u;
            if ((phase == kPhasePos2 || phase == kPhasePos3) && p < cnt && kv != S.T) c = kv > S.T ? 1u : 0u;
            if (c == 1u && jl < L.n) {
                const uint32_t jj = L.off + jl;
                atomicOr((unsigned long long*)&bits[jj >> 6], 1ull << (jj & 63u));
            }
            if (phase == kPhaseKey2) digit = (kv >> kKey4Bits) & ((1u << kFinDigitBits) - 1u);
            if (final_pass) continue;
            hist_add_wave(f.h, digit, c == 2u);
            // compaction in place: every lane has read its record
            const uint64_t bm = wave_ballot(c == 2u);
            if (c == 2u) f.rec[out + lanes_below(bm)] = r;
            out += (uint32_t)__popcll(bm);
        }
        if (final_pass) break;
        cnt = out;
        const bool wide = phase == kPhaseKey2;
        const bool desc = phase == kPhaseKey2 || phase == kPhaseKey3 || phase == kPhaseKey4;
        uint32_t b = 0, bef = 0, count = 0;
        if (!wave_find_bucket(f.h, wide ? kFinBins : phase_bins(phase), desc, S.need, &b, &bef, &count)) {
            S.phase = kPhaseDone;  // inconsistent counts: select no candidate rather than guess
            S.T = 0xFFFFFFFFu;
            S.J = 0;
        } else if (wide) {
            S.need -= bef;
            S.kprefix = (S.kprefix << kFinDigitBits) | b;
            if (S.need == count) {
                S.T = S.kprefix << kKey4Bits;
                S.J = 0xFFFFFFFFu;
                S.phase = kPhaseDone;
            } else {
                S.phase = kPhaseKey4;
            }
        } else {
            advance(S, phase, b, bef, count);
        }
        if (S.phase == kPhasePos1 && L.n <= (1u << 20)) {
            S.jprefix = 0;
            S.phase = kPhasePos2;
        }
    }
    if (lane == 0) f.S = S;
}

// Every remaining digit of layer L from its `cnt` records at grec (the
// filter's: the layer's exact threshold bucket, with full keys), by one
// workgroup: each phase classifies the records left by the previous one,
// marks those its decided prefix selects, histograms and compacts the
// undecided rest, and fixes its digit; the final rule marks what remains
// selected.  The phases and rules are those of the record passes, with key
// bits 17..6 as one digit.  That first phase keeps every record (all are in
// the bucket d1), so it only counts.  The records a later phase keeps are
// those of the bucket the previous search chose, whose count that search
// returned: they go to LDS from the first phase that keeps at most
// kFinLdsRecs, else they are compacted in place.  Once at most kWaveRecs
// remain in LDS, wave 0 finishes alone (finish_wave).
__device__ void finish_records(FinishLds& f, const LayerDesc& L, uint64_t* __restrict__ grec, uint32_t cnt,
                               uint64_t* __restrict__ bits) {
    const uint32_t lane = lane_id(), wave = threadIdx.x / 64;
    bool in_lds = false;
    uint32_t keep = cnt;  // records the next pass keeps
    if (cnt <= kFinLdsRecs) {  // uniform: few enough to work on in LDS from the start
        for (uint32_t p = threadIdx.x; p < cnt; p += kCompactBlock) f.rec[p] = grec[p];
        __syncthreads();
        in_lds = true;
    }
    for (;;) {
        const SelState S = f.S;
        const uint32_t phase = S.phase;
        const bool final_pass = phase == kPhaseDone;
        const bool count_only = phase == kPhaseKey2;
        // where this phase's kept records go: LDS once they are few enough
        const bool to_lds = in_lds || keep <= kFinLdsRecs;
        const uint64_t* src = in_lds ? f.rec : grec;
        uint64_t* dst = to_lds ? f.rec : grec;
        uint32_t out = 0;  // records kept so far (uniform)
        for (uint32_t c0 = 0; c0 < cnt; c0 += kCompactBlock * kFinRecs) {
            // every load at a slot clamped to the last record, all in flight together
            uint64_t r[kFinRecs];
#pragma unroll
            for (int i = 0; i < kFinRecs; ++i) {
                const uint32_t p = c0 + threadIdx.x + i * kCompactBlock;
                r[i] = src[p < cnt ? p : cnt - 1u];
            }
            uint32_t und = 0;  // bit i: record i undecided
#pragma unroll
            for (int i = 0; i < kFinRecs; ++i) {
                const uint32_t p = c0 + threadIdx.x + i * kCompactBlock;
                const uint32_t kv = (uint32_t)(r[i] >> 32), jl = (uint32_t)r[i];
                uint32_t digit = 0;
                uint32_t c = p < cnt ? classify(phase, S, kv, jl, &digit) : 0u;
                // the later position digits' rules assume that only keys equal
                // to T remain, which the pass over position bits 30..20 leaves;
                // where that pass was skipped, the key decides the others here
                if ((phase == kPhasePos2 || phase == kPhasePos3) && p < cnt && kv != S.T) c = kv > S.T ? 1u : 0u;
                if (c == 1u && jl < L.n) {
                    const uint32_t jj = L.off + jl;
                    atomicOr((unsigned long long*)&bits[jj >> 6], 1ull << (jj & 63u));
                }
                if (count_only) digit = (kv >> kKey4Bits) & ((1u << kFinDigitBits) - 1u);
                if (!final_pass) hist_add_wave(f.h, digit, c == 2u);
                if (c == 2u) und |= 1u << i;
            }
            if (final_pass || count_only) continue;
            // compaction: the chunk is in registers once the barrier is
            // passed, and the kept records land below its end (or in LDS)
            uint32_t ws = 0;
#pragma unroll
            for (int i = 0; i < kFinRecs; ++i) ws += (uint32_t)__popcll(wave_ballot((und >> i) & 1u));
            if (lane == 0) f.wsum[wave] = ws;
            __syncthreads();
            uint32_t base = out, total = 0;
            for (uint32_t q = 0; q < (uint32_t)kCompactWaves; ++q) {
                if (q < wave) base += f.wsum[q];
                total += f.wsum[q];
            }
#pragma unroll
            for (int i = 0; i < kFinRecs; ++i) {
                const bool u = (und >> i) & 1u;
                const uint64_t bm = wave_ballot(u);
                const uint32_t slot = base + lanes_below(bm);
                if (u && (!to_lds || slot < kFinLdsRecs)) dst[slot] = r[i];  // (the count fits by construction)
                base += (uint32_t)__popcll(bm);
            }
            out += total;
            __syncthreads();
        }
        if (final_pass) return;
        if (!count_only) {
            cnt = out;
            in_lds = to_lds;
        }
        __syncthreads();  // every wave's counts are in the histogram
        finish_select(f, phase, L, true);
        keep = f.count;
        if (in_lds && cnt <= kWaveRecs) {  // uniform: the rest by one wave
            if (threadIdx.x < 64) finish_wave(f, L, cnt, bits);
            return;
        }
    }
}

// The same from the layer's keys, for a layer whose threshold bucket did not
// fit its record space: each phase reads every key of the layer.
__device__ void finish_keys(FinishLds& f, const LayerDesc& L, const uint16_t* __restrict__ key,
                            const KeySource& ks, uint64_t* __restrict__ bits) {
    const uint32_t w0 = L.off / 64u, w1 = (L.off + L.n + 63u) / 64u;
    for (;;) {
        const SelState S = f.S;
        const uint32_t phase = S.phase;
        key_pass_words<kCompactBlock>(phase, w0, w1, L, S, key, ks, bits, f.h);
        if (phase == kPhaseDone) return;
        __syncthreads();
        finish_select(f, phase, L, false);
    }
}

__global__ __launch_bounds__(kCompactBlock) void k_compact_filter(const TileDesc* __restrict__ tiles, uint32_t parts,
                                                                  const LayerDesc* __restrict__ layers,
                                                                  const SegDesc* __restrict__ lspace,
                                                                  SelState* __restrict__ st,
                                                                  const uint16_t* __restrict__ key, KeySource ks,
                                                                  uint64_t* __restrict__ bits,
                                                                  uint64_t* __restrict__ cand,
                                                                  unsigned long long* __restrict__ ticket,
                                                                  uint32_t* __restrict__ lrec,
                                                                  uint32_t* __restrict__ labove,
                                                                  uint32_t* __restrict__ miss) {
    __shared__ CompactLds lds;
    __shared__ uint32_t s_flag, s_total;
    TileDesc t = tiles[blockIdx.x];
    const int l = t.layer;
    const LayerDesc L = layers[l];
    const SegDesc G = lspace[l];
    const SelState S = st[l];
    uint32_t w0, w1;
    tile_part(t, parts, blockIdx.y, &w0, &w1);
    t.w0 = w0;
    t.w1 = w1;
    t.seg = (uint32_t)l;  // the layer's own record counter
    uint32_t reserved = 0;
    if (w0 < w1) {        // uniform
        if (S.none)       // nothing selected: zero words
            key_pass<false, false, kCompactBlock>(lds.pass, t, L, G, (uint32_t)kDigit1Bins, 1u, 0u, key, bits, lrec,
                                                  cand, labove);
        else if (S.all_bucket)  // the threshold bucket and above, no records
            key_pass<false, false, kCompactBlock>(lds.pass, t, L, G, S.d1, 1u, 0u, key, bits, lrec, cand, labove);
        else  // above the bucket: bits; in it: records with their full keys
            reserved = key_pass<true, false, kCompactBlock, true>(lds.pass, t, L, G, S.d1 + 1u, S.d1, S.d1, key,
                                                                  bits, lrec, cand, labove, nullptr, &ks);
    }
    uint32_t fill = 0;  // the layer's records (all reservations)
    if (!last_of_layer_sum<kCompactBlock>(ticket, l, layer_tiles(L) * parts, reserved, &s_flag, &s_total, &fill))
        return;
    if (S.none || S.phase == kPhaseDone) return;  // the filter wrote the whole mask of the layer
    FinishLds& f = lds.fin;
    if (threadIdx.x == 0) {
        f.S = S;
        if (fill > G.size) {
            f.S.mode = kModeNoRecords;
            atomicOr(miss, 2u);
        }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < kFinBins; b += kCompactBlock) f.h[b] = 0;
    __syncthreads();
    if (fill > G.size)
        finish_keys(f, L, key, ks, bits);
    else
        finish_records(f, L, cand + G.base, fill, bits);
    __syncthreads();
    if (threadIdx.x == 0) st[l] = f.S;
}

hipError_t launch_compact_filter(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, uint32_t parts,
                                 const LayerDesc* layers, const SegDesc* lspace, SelState* st, const uint16_t* key,
                                 const KeySource& ks, uint64_t* bits, uint64_t* cand, unsigned long long* ticket,
                                 uint32_t* lrec, uint32_t* labove, uint32_t* miss) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_compact_filter, dim3(n_tiles, parts), dim3(kCompactBlock), 0, s, tiles, parts, layers, lspace,
                       st, key, ks, bits, cand, ticket, lrec, labove, miss);
    return hipGetLastError();
}


}  // namespace scape
