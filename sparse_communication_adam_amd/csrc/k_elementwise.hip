// k_elementwise.hip - the dense per-element pass and the sparse update pass
// of the SCAPE step, for gfx950 (wave64).
//
// Dense pass (k_ef_compact): one read of every worker's gradient and
// residual, one write of every residual, one read of m, one write of the
// statistic key; at the positions of the current mask it also writes each
// worker's first-moment candidate into that worker's compacted sparse buffer.
// Lane l of a wave handles element l of each 64-element word, so every load
// and store of a wave is one contiguous 128- or 256-byte segment, the mask
// word is a wave-uniform scalar, and a masked element's slot in the sparse
// buffer is block_prefix[word] + (set bits of the word below the lane), a
// single mbcnt.  The first radix digit of the key is histogrammed in LDS per
// tile and flushed once per tile.
//
// Sparse pass (k_reduce_update): one lane per masked position: the W-way mean
// of the sparse buffers in worker order, the reconstruction of the averaged
// gradient from that one buffer, the AdamS normaliser, and the m/v/x update.
//
// The operations follow the SCAPE step of "SCAPE: Accurate and Efficient LLM
// Training with Extreme Sparse Communication" as stated in include/scape.h
// (error feedback: gist.science Technical Summary s.1 and s.2 Key Design
// Insights; first-moment statistics: shd-paper.top abstract; single-buffer
// reconstruction: Technical Summary s.2).  All fp32, round to nearest even,
// compiled with -ffp-contract=off so no multiply-add is fused.
#include "scape_device.h"

namespace scape {

// Workers are processed in chunks of up to kWorkerChunk; within a chunk every
// load is issued before any store, so a wave keeps E words x chunk x (fp32 r,
// bf16 g) in flight.  WT > 0 fixes the worker count at compile time.
constexpr int kWorkerChunk = 4;

// One wave-iteration of the dense pass over words [w0, w0+E).  GUARD = false
// is the interior case (all E words inside the tile and the layer), with no
// per-element predicate; GUARD = true handles a layer's last, partial words.
// Lane addresses are one 64-bit base per array plus compile-time offsets of
// 64 elements per word.
template <int WT, bool GUARD>
__device__ __forceinline__ void ef_iteration(uint32_t w0, uint32_t w1, uint32_t lend, int owner, int W,
                                             const WorkerPtrs& wp, float b1, float c1, const float* __restrict__ m,
                                             const uint64_t* __restrict__ cur_bits,
                                             const uint32_t* __restrict__ cur_prefix, uint32_t k_cap,
                                             uint32_t* __restrict__ key, uint32_t* h) {
    constexpr int E = kWordsPerWaveIter;
    const uint32_t lane = lane_id();
    const size_t j0 = (size_t)w0 * 64u + lane;
    uint64_t word[E];
    uint32_t pre[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t wc = GUARD ? min(w0 + e, w1 - 1) : w0 + e;
        word[e] = cur_bits[wc];
        pre[e] = cur_prefix[wc];
    }
    bool inl[E];
#pragma unroll
    for (int e = 0; e < E; ++e) inl[e] = GUARD ? (w0 + e < w1) && (j0 + 64u * e < lend) : true;
    float bm[E];
    const float* mp = m + j0;
#pragma unroll
    for (int e = 0; e < E; ++e) bm[e] = inl[e] ? mp[64 * e] : 0.0f;
    uint32_t rank[E], kk[E];
    bool msk[E];
    uint64_t any = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        bm[e] = b1 * bm[e];
        rank[e] = pre[e] + lanes_below(word[e]);
        msk[e] = inl[e] && ((word[e] >> lane) & 1ull) && rank[e] < k_cap;
        kk[e] = 0;
        any |= word[e];
    }
    for (int i0 = 0; i0 < W; i0 += kWorkerChunk) {
        float rv[kWorkerChunk][E];
        uint16_t gv[kWorkerChunk][E];
#pragma unroll
        for (int c = 0; c < kWorkerChunk; ++c) {
            if (i0 + c >= W) break;
            const float* rp = wp.r[i0 + c] + j0;
            const uint16_t* gp = wp.g[i0 + c] + j0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                rv[c][e] = inl[e] ? rp[64 * e] : 0.0f;
                gv[c][e] = inl[e] ? gp[64 * e] : (uint16_t)0;
            }
        }
#pragma unroll
        for (int c = 0; c < kWorkerChunk; ++c) {
            const int i = i0 + c;
            if (i >= W) break;
            float* rp = wp.r[i] + j0;
            float mt[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float a = rv[c][e] + bf16_bits_to_f32(gv[c][e]);
                mt[e] = bm[e] + c1 * a;
                if (i == owner) kk[e] = magnitude_key(mt[e]);
                if (inl[e]) rp[64 * e] = msk[e] ? 0.0f : a;
            }
            if (any) {  // wave-uniform: most iterations of a sparse mask skip this
                float* __restrict__ b = wp.b[i];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (msk[e]) b[rank[e]] = mt[e];
            }
        }
    }
    uint32_t* kp = key + j0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (inl[e]) kp[64 * e] = kk[e];
        hist_add_wave(h, kk[e] >> (31 - kDigit1Bits), inl[e]);
    }
}

template <int WT>
__global__ __launch_bounds__(kBlock) void k_ef_compact(const TileDesc* __restrict__ tiles,
                                                       const LayerDesc* __restrict__ layers, WorkerPtrs wp,
                                                       StepScalars sc, const float* __restrict__ m,
                                                       const uint64_t* __restrict__ cur_bits,
                                                       const uint32_t* __restrict__ cur_prefix, uint32_t k_cap,
                                                       uint32_t* __restrict__ key, uint32_t* __restrict__ hist) {
    constexpr int E = kWordsPerWaveIter;
    __shared__ uint32_t h[kDigit1Bins];
    for (int b = threadIdx.x; b < kDigit1Bins; b += kBlock) h[b] = 0;
    __syncthreads();

    const TileDesc t = tiles[blockIdx.x];
    const LayerDesc L = layers[t.layer];
    const uint32_t lend = L.off + L.n;
    const uint32_t wave = threadIdx.x / 64;
    const int W = WT > 0 ? WT : sc.W;
    // words [t.w0, full_end) lie wholly inside the layer
    const uint32_t full_end = min(t.w1, lend / 64u);
    for (uint32_t w0 = t.w0 + wave * E; w0 < t.w1; w0 += kWaves * E) {
        if (w0 + E <= full_end)
            ef_iteration<WT, false>(w0, t.w1, lend, L.owner, W, wp, sc.beta1, sc.c1, m, cur_bits, cur_prefix, k_cap,
                                    key, h);
        else
            ef_iteration<WT, true>(w0, t.w1, lend, L.owner, W, wp, sc.beta1, sc.c1, m, cur_bits, cur_prefix, k_cap,
                                   key, h);
    }
    __syncthreads();
    hist_flush(h, hist + (size_t)t.layer * kHistBins, kDigit1Bins);
}

hipError_t launch_ef_compact(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                             const WorkerPtrs& wp, const StepScalars& sc, const float* m, const uint64_t* cur_bits,
                             const uint32_t* cur_prefix, uint32_t k_cap, uint32_t* key, uint32_t* hist) {
    if (n_tiles == 0) return hipSuccess;
#define SCAPE_EF_CASE(WV)                                                                                       \
    case WV:                                                                                                    \
        hipLaunchKernelGGL(k_ef_compact<WV>, dim3(n_tiles), dim3(kBlock), 0, s, tiles, layers, wp, sc, m, cur_bits, \
                           cur_prefix, k_cap, key, hist);                                                       \
        break;
    switch (sc.W) {
        SCAPE_EF_CASE(1)
        SCAPE_EF_CASE(2)
        SCAPE_EF_CASE(3)
        SCAPE_EF_CASE(4)
        SCAPE_EF_CASE(8)
        SCAPE_EF_CASE(16)
        SCAPE_EF_CASE(32)
        default:
            hipLaunchKernelGGL(k_ef_compact<0>, dim3(n_tiles), dim3(kBlock), 0, s, tiles, layers, wp, sc, m, cur_bits,
                               cur_prefix, k_cap, key, hist);
    }
#undef SCAPE_EF_CASE
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_reduce_update(WorkerPtrs wp, StepScalars sc, float* __restrict__ x,
                                                          float* __restrict__ m, float* __restrict__ v,
                                                          const uint32_t* __restrict__ idx,
                                                          const uint32_t* __restrict__ prefix, uint32_t n_words,
                                                          uint32_t n_pad, uint32_t k_cap) {
    const uint32_t total = prefix[n_words];
    const uint32_t cnt = total < k_cap ? total : k_cap;
    const int W = sc.W;
    const float fW = (float)W;
    for (uint32_t q = blockIdx.x * kBlock + threadIdx.x; q < cnt; q += gridDim.x * kBlock) {
        const uint32_t jj = idx[q];
        if (jj >= n_pad) continue;
        float s = wp.b[0][q];
        for (int i = 1; i < W; ++i) s = s + wp.b[i][q];
        const float bb = s / fW;
        const float mo = m[jj];
        const float ghat = (bb - sc.beta1 * mo) / sc.c1;
        const float vv = sc.beta2 * (mo * mo) + sc.c2 * (ghat * ghat);
        v[jj] = vv;
        m[jj] = bb;
        const float xv = x[jj];
        float u = bb / (sqrtf(vv) + sc.eps);
        if (sc.wd != 0.0f) u = u + sc.wd * xv;
        x[jj] = xv - sc.lr * u;
    }
}

hipError_t launch_reduce_update(hipStream_t s, const WorkerPtrs& wp, const StepScalars& sc, float* x, float* m,
                                float* v, const uint32_t* cur_idx, const uint32_t* cur_prefix, uint32_t n_words,
                                uint32_t n_pad, uint32_t k_cap) {
    if (k_cap == 0) return hipSuccess;
    uint32_t blocks = (k_cap + kBlock - 1) / kBlock;
    if (blocks > 16384u) blocks = 16384u;
    hipLaunchKernelGGL(k_reduce_update, dim3(blocks), dim3(kBlock), 0, s, wp, sc, x, m, v, cur_idx, cur_prefix,
                       n_words, n_pad, k_cap);
    return hipGetLastError();
}

// Statistic keys and the first-digit histogram from a given m-tilde (the
// standalone mask build).
__global__ __launch_bounds__(kBlock) void k_keys_from_mtilde(const TileDesc* __restrict__ tiles,
                                                             const LayerDesc* __restrict__ layers,
                                                             const float* __restrict__ mtilde,
                                                             uint32_t* __restrict__ key,
                                                             uint32_t* __restrict__ hist) {
    __shared__ uint32_t h[kDigit1Bins];
    for (int b = threadIdx.x; b < kDigit1Bins; b += kBlock) h[b] = 0;
    __syncthreads();
    const TileDesc t = tiles[blockIdx.x];
    const LayerDesc L = layers[t.layer];
    const uint32_t lend = L.off + L.n;
    const uint32_t lane = lane_id();
    const uint32_t wave = threadIdx.x / 64;
    for (uint32_t w0 = t.w0 + wave * kWordsPerWaveIter; w0 < t.w1; w0 += kWaves * kWordsPerWaveIter) {
        uint32_t kk[kWordsPerWaveIter];
        bool inl[kWordsPerWaveIter];
#pragma unroll
        for (int e = 0; e < kWordsPerWaveIter; ++e) {
            const uint32_t wi = w0 + e;
            const uint32_t jj = wi * 64u + lane;
            inl[e] = wi < t.w1 && jj < lend;
            kk[e] = inl[e] ? magnitude_key(mtilde[jj]) : 0u;
        }
#pragma unroll
        for (int e = 0; e < kWordsPerWaveIter; ++e) {
            const uint32_t jj = (w0 + e) * 64u + lane;
            if (inl[e]) key[jj] = kk[e];
            hist_add_wave(h, kk[e] >> (31 - kDigit1Bits), inl[e]);
        }
    }
    __syncthreads();
    hist_flush(h, hist + (size_t)t.layer * kHistBins, kDigit1Bins);
}

hipError_t launch_keys_from_mtilde(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                                   const float* mtilde, uint32_t* key, uint32_t* hist) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_keys_from_mtilde, dim3(n_tiles), dim3(kBlock), 0, s, tiles, layers, mtilde, key, hist);
    return hipGetLastError();
}

struct BufPtrs {
    const float* b[SCAPE_MAX_WORKERS];
};

__global__ __launch_bounds__(kBlock) void k_reduce_sparse(BufPtrs bp, int32_t W, uint64_t k, float* __restrict__ out) {
    const float fW = (float)W;
    for (uint64_t q = (uint64_t)blockIdx.x * kBlock + threadIdx.x; q < k; q += (uint64_t)gridDim.x * kBlock) {
        float s = bp.b[0][q];
        for (int i = 1; i < W; ++i) s = s + bp.b[i][q];
        out[q] = s / fW;
    }
}

hipError_t launch_reduce_sparse(hipStream_t s, const float* const* bufs, int32_t W, int64_t k, float* out) {
    if (k <= 0) return hipSuccess;
    BufPtrs bp{};
    for (int i = 0; i < W; ++i) bp.b[i] = bufs[i];
    uint64_t blocks = ((uint64_t)k + kBlock - 1) / kBlock;
    if (blocks > 16384u) blocks = 16384u;
    hipLaunchKernelGGL(k_reduce_sparse, dim3((uint32_t)blocks), dim3(kBlock), 0, s, bp, W, (uint64_t)k, out);
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_fill_u32(uint32_t* __restrict__ p, uint64_t n, uint32_t value) {
    for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (uint64_t)gridDim.x * kBlock)
        p[i] = value;
}

hipError_t launch_fill_u32(hipStream_t s, uint32_t* p, uint64_t n, uint32_t value) {
    if (n == 0) return hipSuccess;
    uint64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 8192u) blocks = 8192u;
    hipLaunchKernelGGL(k_fill_u32, dim3((uint32_t)blocks), dim3(kBlock), 0, s, p, n, value);
    return hipGetLastError();
}

}  // namespace scape
