// k_elementwise.hip - the dense per-element pass and the sparse update pass
// of the SCAPE step, for gfx950 (wave64).
//
// Dense pass (k_ef_compact): one read of every worker's gradient and
// residual, one write of every residual, one read of m, one write of the top
// 16 bits of the statistic key (the full key only on request); at the
// positions of the current mask it also writes each worker's first-moment
// candidate into that worker's compacted sparse buffer.
// Lane l of a wave handles element l of each 64-element word, so every load
// and store of a wave is one contiguous 128- or 256-byte segment, the mask
// word is a wave-uniform scalar, and a masked element's slot in the sparse
// buffer is block_prefix[word] + (set bits of the word below the lane), a
// single mbcnt.
//
// Dense AdamS pass (k_dense_adams): the comparison baseline, the same one-shot
// layout as the dense SCAPE pass: the W gradients averaged in worker order and
// the AdamS update of x, m, v on every element.
//
// Sparse pass (k_reduce_update): eight masked positions per lane: the W-way mean
// of the sparse buffers in worker order, the reconstruction of the averaged
// gradient from that one buffer, the AdamS normaliser, and the m/v/x update.
// The dense pass leaves m of every masked position in a compacted stash, so
// the sparse pass gathers only x.
//
// The operations follow the SCAPE step of "SCAPE: Accurate and Efficient LLM
// Training with Extreme Sparse Communication" as stated in include/scape.h
// (error feedback: gist.science Technical Summary s.1 and s.2 Key Design
// Insights; first-moment statistics: shd-paper.top abstract; single-buffer
// reconstruction: Technical Summary s.2).  All fp32, round to nearest even,
// compiled with -ffp-contract=off so no multiply-add is fused.
#include "scape_device.h"

namespace scape {

// Dense pass, one-shot layout: a wave handles a short run of consecutive
// 64-element words (how many depends on W, below) and exits; a workgroup's
// four waves take consecutive runs.  Work is dispatched in address order, so
// the words in flight at any time are a compact window of every array; on
// MI355X that sustains a higher HBM rate than long-lived workgroups streaming
// separate tiles or striding over the grid.  Per word, a
// 16-bit descriptor gives the owner worker (bits 8..13) and the number of
// elements of the word inside its layer (bits 0..6, 1..64; 0 = padding).
// Every worker's loads are issued before any store.
// The dense pass loads and stores its streamed arrays (gradients,
// residuals, m, keys) non-temporally, and writes the sparse buffers and the
// m stash, which the update pass reads next, through the caches.  The
// streamed stores matter most: with plain residual and key stores the pass
// ran at 0.87 of a pass that only moves the same bytes over the same buffers
// in a fresh GPU's first process, with non-temporal ones at 0.96-1.0
// (1.75B shape: 14.5 against 13.0 ms); non-temporal stores to the sparse
// buffers made the update slower.
template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
    return __builtin_nontemporal_load(p);
}

#ifndef SCAPE_EF_BLOCK
#define SCAPE_EF_BLOCK 256
#endif
constexpr int kEfBlock = SCAPE_EF_BLOCK;  // threads per workgroup of the dense pass
constexpr int kEfWaves = kEfBlock / 64;
// Each XCD streams one contiguous eighth of the words (measured: the dense
// pass 0.3-0.9 ms faster on the 1.75B workload, most where the process's
// buffers map worst).
#ifndef SCAPE_EF_XCD
#define SCAPE_EF_XCD 1
#endif
constexpr bool kEfXcd = SCAPE_EF_XCD != 0;
// The exception: at W = 4 in the interleaved layout with the update inside,
// measured build against build on one state, the pass without the
// renumbering took 14.02-14.04 against 14.21-14.24 ms in a fresh GPU's first
// process (where a training job's process runs) and 13.75 against 13.52 in
// the process after it; at W = 8 and 32 the renumbering was 4-13% faster in
// either.
template <int WT, int UPD>
constexpr bool ef_xcd() {
    return kEfXcd && !(WT == 4 && UPD == 2);
}

// Consecutive words per wave.  Measured on the 1.75B shape in both
// residual/gradient layouts: at W = 4 one word per wave took 15.3 ms (one
// array per worker) and 14.3 ms (worker-interleaved) where two took 15.4 and
// 14.7 and four 15.5 and 15.1; at W = 8 (0.35B shape) one word 6.04 / 5.67 ms
// against 6.08 / 5.81 with two.  At W = 32 one and two words were within 1%
// of each other.  At W = 1 (640 bytes per word) the per-word descriptor, mask
// word and prefix loads weigh more: eight words per wave took 5.0 ms, two
// 5.9 ms.
#ifndef SCAPE_EF_W1
#define SCAPE_EF_W1 8
#endif
template <int WT>
constexpr uint32_t ef_words() {
    return WT == 1 ? SCAPE_EF_W1 : 1;
}

// Threads per workgroup.  At W = 8 one-wave workgroups are faster, measured
// build against build on one state: 64, 128 and 256 threads took 7.94, 8.08
// and 8.18 ms on the 0.55B shape (update inside), 6.59, 6.66 and 6.69-6.70
// on the GPT-345M shape (x, v and m streamed whole) and 5.23, 5.31 and 5.35
// there without the update.  At W = 32 256 threads were the fastest (64:
// 20.99, 128: 20.63, 256: 20.44 ms on the adversarial shard); at W = 4 and
// W = 1 (1.75B shape) the three were within 0.5%.
#ifndef SCAPE_EF_BLOCK_W8
#define SCAPE_EF_BLOCK_W8 64
#endif
template <int WT>
constexpr int ef_block() {
    return WT == 8 ? SCAPE_EF_BLOCK_W8 : kEfBlock;
}

// With UPD the pass also finishes the step at the current mask's positions:
// it has every worker's candidate of an element in registers, so the W-way
// mean of what the workers send, the reconstruction and the m / v / x update
// (the same fp32 operations in the same order as k_reduce_update) need no
// second pass over the sparse buffers.  UPD 1 and 3: x and v are separate
// arrays; UPD 2 and 4: x holds (x, v) pairs.  UPD 1 and 2 (sparse masks):
// only masked lanes touch x, v and m; the x load of a masked lane is issued
// as soon as its mask word is known, beside the element loads, and every
// other lane loads `dummy`, which nothing writes.  UPD 3 and 4 (denser
// masks, where most lines of x, v and m hold a masked element anyway): every
// lane writes x, v and m back, the old values where it is not masked, so
// those arrays move as whole lines instead of scattered partial ones.  UPD 3
// streams x and v in with the element loads.  UPD 4 loads and stores the
// (x, v) pairs of a 16-element group (one 128-byte line) only where the
// group holds a masked element, issued once the mask word is known (at a
// kept fraction of 1/10 about one line in five is skipped: the GPT-345M
// shape's pass 6.33 against 6.57 ms, build against build on one state).
template <int WT, bool K32, int UPD>
__global__ __launch_bounds__(ef_block<WT>()) void k_ef_compact(const uint16_t* __restrict__ word_info, uint32_t n_words,
                                                       WorkerPtrs wp, StepScalars sc, float* __restrict__ m,
                                                       const uint64_t* __restrict__ cur_bits,
                                                       const uint32_t* __restrict__ cur_prefix, uint32_t k_cap,
                                                       uint16_t* __restrict__ key16, uint32_t* __restrict__ key32,
                                                       float* __restrict__ m_stash, uint32_t* __restrict__ clear,
                                                       uint32_t n_clear, float* __restrict__ x, float* __restrict__ v,
                                                       const float* __restrict__ dummy) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    constexpr int WMAX = WT > 0 ? WT : SCAPE_MAX_WORKERS;
    constexpr uint32_t kWords = ef_words<WT>();
    constexpr int kB = ef_block<WT>(), kNW = kB / 64;
    // the selection's histogram rows, zeroed on the way (spread over every
    // workgroup; a few KB per layer)
    for (uint32_t i = blockIdx.x * kB + threadIdx.x; i < n_clear; i += gridDim.x * kB) clear[i] = 0u;
    const uint32_t blk = ef_xcd<WT, UPD>() ? xcd_block(blockIdx.x, gridDim.x) : blockIdx.x;
    // wave-uniform, so the descriptors below are scalar loads
    const uint32_t w0 = (blk * kNW + __builtin_amdgcn_readfirstlane(threadIdx.x / 64)) * kWords;
    if (w0 >= n_words) return;
    const uint32_t lane = lane_id();
    const int W = WT > 0 ? WT : sc.W;
    // every array holds n_pad elements, so all 64 lanes of a word may load:
    // the element loads of all the wave's words (clamped to the last word) go
    // out at once, beside the words' descriptors, and the padding lanes are
    // dropped only before the stores
    float mo[kWords];
    float rv[kWords][WMAX];
    uint16_t gv[kWords][WMAX];
    constexpr bool kPairs = UPD == 2 || UPD == 4;  // x holds (x, v) pairs
    constexpr bool kFull = UPD >= 3;                // every lane stores x, v and m
    float x0[kWords], v0[kWords];
    f32x2* __restrict__ xv = reinterpret_cast<f32x2*>(x);
#pragma unroll
    for (uint32_t e = 0; e < kWords; ++e) {
        const size_t wc = min(w0 + e, n_words - 1u);
        const size_t j = wc * 64u + lane, jw = wc * wp.ws + lane;
        mo[e] = stream_load(&m[j]);
#pragma unroll
        for (int i = 0; i < WMAX; ++i) {
            if (i >= W) break;
            rv[e][i] = stream_load(&wp.r[i][jw]);
            gv[e][i] = stream_load(&wp.g[i][jw]);
        }
        if (kFull && !kPairs) {
            x0[e] = stream_load(&x[j]);
            v0[e] = stream_load(&v[j]);
        }
    }
    // the (x, v) pairs of the lines that hold a masked element (UPD 4), or
    // the parameters of the masked lanes (UPD 1, 2), loaded once the element
    // loads are out (the scheduling barrier keeps the wait for the mask word
    // behind them); the other lanes load `dummy`
    if (kFull && kPairs) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t e = 0; e < kWords; ++e) {
            const uint32_t wc = min(w0 + e, n_words - 1u);
            const uint64_t word = cur_bits[wc];
            const bool line = ((word >> (lane & ~15u)) & 0xFFFFull) != 0ull;
            const size_t j = (size_t)wc * 64u + lane;
            const f32x2 p = stream_load(line ? &xv[j] : reinterpret_cast<const f32x2*>(dummy));
            x0[e] = p.x;
            v0[e] = p.y;
        }
    }
    if (UPD && !kFull) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t e = 0; e < kWords; ++e) {
            const uint32_t wc = min(w0 + e, n_words - 1u);
            const uint64_t word = cur_bits[wc];
            const uint32_t rank = cur_prefix[wc] + lanes_below(word);
            const bool msk = ((word >> lane) & 1ull) && rank < k_cap && w0 + e < n_words;
            const size_t j = (size_t)wc * 64u + lane;
            if (UPD == 2)
                x0[e] = (msk ? reinterpret_cast<const f32x2*>(&xv[j]) : reinterpret_cast<const f32x2*>(dummy))->x;
            else
                x0[e] = *(msk ? &x[j] : dummy);
        }
    }
#pragma unroll
    for (uint32_t e = 0; e < kWords; ++e) {
        const uint32_t w = w0 + e;
        if (w >= n_words) break;
        const size_t j = (size_t)w * 64u + lane, jw = (size_t)w * wp.ws + lane;
        const uint32_t info = word_info[w];
        const uint64_t word = cur_bits[w];
        const uint32_t pre = cur_prefix[w];
        const uint32_t count = info & 127u;
        const int owner = (int)((info >> 8) & 63u);
        // padding lanes of a layer's last word store nothing (their mask bits
        // are clear); the test guards the stores only, so that no load waits
        // for the descriptor
        const bool live = lane < count;
        const uint32_t rank = pre + lanes_below(word);
        const bool msk = ((word >> lane) & 1ull) && rank < k_cap;
        const float bm = sc.beta1 * mo[e];
        uint32_t kk = 0;
        float s = 0.0f;  // the sum of what the workers send, in worker order
#pragma unroll
        for (int i = 0; i < WMAX; ++i) {
            if (i >= W) break;
            const float a = rv[e][i] + bf16_bits_to_f32(gv[e][i]);
            const float mt = bm + sc.c1 * a;
            if (i == owner) kk = magnitude_key(mt);
            if (live) __builtin_nontemporal_store(msk ? 0.0f : a, &wp.r[i][jw]);
            if (msk) wp.b[i][rank] = mt;
            if (UPD) s = i == 0 ? mt : s + mt;
        }
        // the selection reads the top 16 bits; candidates get their full key
        // back from the state (or from key32 when it is asked for)
        if (live) __builtin_nontemporal_store((uint16_t)(kk >> kKeyShift), &key16[j]);
        if (K32 && live) key32[j] = kk;
        if (!UPD) {
            // m before the step, compacted like the sparse buffers: the update
            // pass reads it contiguously instead of gathering one line per position
            if (msk) m_stash[rank] = mo[e];
        } else if (kFull) {
            // every lane computes; the unmasked ones store what they loaded
            const float bb = s / (float)W;
            const float ghat = (bb - bm) / sc.c1;
            const float vv = sc.beta2 * (mo[e] * mo[e]) + sc.c2 * (ghat * ghat);
            float upd = bb / (sqrtf(vv) + sc.eps);
            if (sc.wd != 0.0f) upd = upd + sc.wd * x0[e];
            const float xn = x0[e] - sc.lr * upd;
            if (live) {
                __builtin_nontemporal_store(msk ? bb : mo[e], &m[j]);
                if (kPairs) {
                    const bool line = ((word >> (lane & ~15u)) & 0xFFFFull) != 0ull;
                    f32x2 p;
                    p.x = msk ? xn : x0[e];
                    p.y = msk ? vv : v0[e];
                    if (line) __builtin_nontemporal_store(p, &xv[j]);
                } else {
                    __builtin_nontemporal_store(msk ? xn : x0[e], &x[j]);
                    __builtin_nontemporal_store(msk ? vv : v0[e], &v[j]);
                }
            }
        } else if (msk) {
            const float bb = s / (float)W;
            const float ghat = (bb - bm) / sc.c1;
            const float vv = sc.beta2 * (mo[e] * mo[e]) + sc.c2 * (ghat * ghat);
            float upd = bb / (sqrtf(vv) + sc.eps);
            if (sc.wd != 0.0f) upd = upd + sc.wd * x0[e];
            __builtin_nontemporal_store(bb, &m[j]);
            if (UPD == 2) {
                f32x2 p;
                p.x = x0[e] - sc.lr * upd;
                p.y = vv;
                xv[j] = p;
            } else {
                __builtin_nontemporal_store(vv, &v[j]);
                x[j] = x0[e] - sc.lr * upd;
            }
        }
    }
}

// Worker lanes (worker-interleaved arrays, W = 4, no update in the pass, no
// full keys asked for): a wave's lanes split into W groups of 64 / W, a
// group per worker, and each lane takes W consecutive elements of its
// worker's part of the word, which in the interleaved layout are the lane's
// own 4W (residuals) or 2W (gradients) bytes of the word.  Every array then
// moves as one access per lane of 4W bytes (residuals; m, whose same
// elements every group reads), 2W (gradients) or 2W (keys, stored by the
// owner's group) instead of W accesses of 4 or 2 bytes: the same bytes in a
// quarter of the memory instructions.  The arithmetic and its order per
// element and worker are those above.  (At W = 8 the same mapping was much
// slower on the 0.35B and 0.55B shapes: every lane then reads 32 bytes of m
// that seven other groups read too.  With the update in the pass it was no
// faster than the mapping above, whether the workers' candidates met through
// lane shuffles or through LDS.)
#ifndef SCAPE_EF_WL
#define SCAPE_EF_WL 1
#endif
template <int W>
__global__ __launch_bounds__(kEfBlock) void k_ef_wl(const uint16_t* __restrict__ word_info, uint32_t n_words,
                                                  WorkerPtrs wp, StepScalars sc, const float* __restrict__ m,
                                                  const uint64_t* __restrict__ cur_bits,
                                                  const uint32_t* __restrict__ cur_prefix, uint32_t k_cap,
                                                  uint16_t* __restrict__ key16, float* __restrict__ m_stash,
                                                  uint32_t* __restrict__ clear, uint32_t n_clear) {
    typedef float fvec __attribute__((ext_vector_type(W)));
    typedef uint16_t hvec __attribute__((ext_vector_type(W)));
    constexpr uint32_t kLanesPerWorker = 64 / W;
    for (uint32_t i = blockIdx.x * kEfBlock + threadIdx.x; i < n_clear; i += gridDim.x * kEfBlock) clear[i] = 0u;
    const uint32_t blk = kEfXcd ? xcd_block(blockIdx.x, gridDim.x) : blockIdx.x;
    const uint32_t w = blk * kEfWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    if (w >= n_words) return;
    const uint32_t lane = lane_id();
    const uint32_t wi = lane / kLanesPerWorker, q = lane % kLanesPerWorker;
    // worker wi's q-th group of W elements of word w: in the interleaved
    // layout (word stride 64 W, worker i at 64 i) that is element w * 64 W +
    // lane * W of the array worker 0's pointer starts
    float* rp = wp.r[0] + (size_t)w * (64u * W) + lane * W;
    const uint16_t* gp = wp.g[0] + (size_t)w * (64u * W) + lane * W;
    const fvec rv = stream_load(reinterpret_cast<const fvec*>(rp));
    const hvec gv = stream_load(reinterpret_cast<const hvec*>(gp));
    // the group's sparse buffer, chosen among the workers' pointers held in
    // scalar registers (the empty statements keep the compiler from turning
    // the choice into a per-lane load of the argument block)
    float* bp;
    {
        float* bs[W];
#pragma unroll
        for (int i = 0; i < W; ++i) {
            bs[i] = wp.b[i];
            asm volatile("" : "+s"(bs[i]));
        }
        bp = bs[0];
#pragma unroll
        for (int i = 1; i < W; ++i) bp = wi == (uint32_t)i ? bs[i] : bp;
    }
    const fvec mv = stream_load(reinterpret_cast<const fvec*>(m + (size_t)w * 64u + q * W));
    const uint32_t info = word_info[w];
    const uint64_t word = cur_bits[w];
    const uint32_t pre = cur_prefix[w];
    const uint32_t count = info & 127u;
    const uint32_t owner = (info >> 8) & 63u;
    // the lane's W mask bits, and the set bits of the word before them
    const uint32_t p0 = q * W;
    const uint32_t slice = (uint32_t)(word >> p0) & ((1u << W) - 1u);
    const uint32_t below = pre + (uint32_t)__popcll(word & ((1ull << p0) - 1ull));
    fvec out;
    hvec kout;
#pragma unroll
    for (int e = 0; e < W; ++e) {
        const bool live = p0 + e < count;  // padding elements keep their residual
        const uint32_t rank = below + (uint32_t)__popc(slice & ((1u << e) - 1u));
        const bool msk = ((slice >> e) & 1u) && rank < k_cap;
        const float bm = sc.beta1 * mv[e];
        const float a = rv[e] + bf16_bits_to_f32(gv[e]);
        const float mt = bm + sc.c1 * a;
        out[e] = live ? (msk ? 0.0f : a) : rv[e];
        kout[e] = live ? (uint16_t)(magnitude_key(mt) >> kKeyShift) : (uint16_t)0;
        if (msk) {
            bp[rank] = mt;
            if (wi == 0) m_stash[rank] = mv[e];
        }
    }
    __builtin_nontemporal_store(out, reinterpret_cast<fvec*>(rp));
    if (wi == owner) __builtin_nontemporal_store(kout, reinterpret_cast<hvec*>(key16 + (size_t)w * 64u + q * W));
}

hipError_t launch_ef_compact(hipStream_t s, const uint16_t* word_info, uint32_t n_words, const WorkerPtrs& wp,
                             const StepScalars& sc, float* m, const uint64_t* cur_bits,
                             const uint32_t* cur_prefix, uint32_t k_cap, uint16_t* key16, uint32_t* key32,
                             float* m_stash, uint32_t* clear, uint32_t n_clear, int upd, float* x, float* v,
                             const float* dummy) {
    if (n_words == 0) return n_clear ? launch_fill_u32(s, clear, n_clear, 0u) : hipSuccess;
    const dim3 block(kEfBlock);
    if (SCAPE_EF_WL && upd == 0 && !key32 && sc.W == 4 && wp.ws == 64u * 4u) {
        hipLaunchKernelGGL(k_ef_wl<4>, dim3((n_words + kEfWaves - 1) / kEfWaves), block, 0, s, word_info, n_words, wp,
                           sc, m, cur_bits, cur_prefix, k_cap, key16, m_stash, clear, n_clear);
        return hipGetLastError();
    }
#define SCAPE_EF_LAUNCH(WV, K, U)                                                                                  \
    hipLaunchKernelGGL((k_ef_compact<WV, K, U>),                                                                   \
                       dim3((n_words + ef_block<WV>() / 64 * ef_words<WV>() - 1) /                                  \
                            (ef_block<WV>() / 64 * ef_words<WV>())),                                                \
                       dim3(ef_block<WV>()), 0, s,                                                                  \
                       word_info, n_words, wp, sc, m, cur_bits, cur_prefix, k_cap, key16, key32, m_stash, clear,   \
                       n_clear, x, v, dummy)
#define SCAPE_EF_UPD(WV, K)                          \
    switch (upd) {                                   \
        case 1: SCAPE_EF_LAUNCH(WV, K, 1); break;    \
        case 2: SCAPE_EF_LAUNCH(WV, K, 2); break;    \
        case 3: SCAPE_EF_LAUNCH(WV, K, 3); break;    \
        case 4: SCAPE_EF_LAUNCH(WV, K, 4); break;    \
        default: SCAPE_EF_LAUNCH(WV, K, 0); break;   \
    }
#define SCAPE_EF_CASE(WV)                     \
    case WV:                                  \
        if (key32) SCAPE_EF_UPD(WV, true)     \
        else SCAPE_EF_UPD(WV, false)          \
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
            if (key32) SCAPE_EF_UPD(0, true)
            else SCAPE_EF_UPD(0, false)
    }
#undef SCAPE_EF_LAUNCH
#undef SCAPE_EF_UPD
#undef SCAPE_EF_CASE
    return hipGetLastError();
}

// Dense AdamS step: consecutive 64-element words per wave, four waves per
// workgroup, every load of the wave's words issued before any descriptor is
// consulted (all arrays hold n_pad elements); the padding lanes of a layer's
// last word store nothing.  A word loads 512 + 128 W bytes; the words per
// wave keep about 2 KB in flight (measured at W = 4: 8.6 ms per step with one
// word per wave, 8.0 with two, 8.2 with four).
template <int WT>
constexpr uint32_t da_words() {
    return (WT == 1 || WT == 2) ? 4 : (WT >= 3 && WT <= 8) ? 2 : 1;
}

template <int WT>
__global__ __launch_bounds__(kBlock) void k_dense_adams(const uint16_t* __restrict__ word_info, uint32_t n_words,
                                                        WorkerPtrs wp, StepScalars sc, float* __restrict__ x,
                                                        float* __restrict__ m, float* __restrict__ v) {
    constexpr int WMAX = WT > 0 ? WT : SCAPE_MAX_WORKERS;
    constexpr uint32_t kDaWords = da_words<WT>();
    const uint32_t w0 = (blockIdx.x * kWaves + threadIdx.x / 64) * kDaWords;
    if (w0 >= n_words) return;
    const uint32_t lane = lane_id();
    const int W = WT > 0 ? WT : sc.W;
    // every array is streamed once: non-temporal loads and stores (measured
    // 8.5 against 8.7-8.9 ms per step on the 1.75B workload)
    float mo[kDaWords], xo[kDaWords];
    uint16_t gv[kDaWords][WMAX];
#pragma unroll
    for (uint32_t e = 0; e < kDaWords; ++e) {
        const size_t wc = min(w0 + e, n_words - 1u);
        const size_t j = wc * 64u + lane, jw = wc * wp.ws + lane;
        mo[e] = stream_load(&m[j]);
        xo[e] = stream_load(&x[j]);
#pragma unroll
        for (int i = 0; i < WMAX; ++i) {
            if (i >= W) break;
            gv[e][i] = stream_load(&wp.g[i][jw]);
        }
    }
#pragma unroll
    for (uint32_t e = 0; e < kDaWords; ++e) {
        const uint32_t w = w0 + e;
        if (w >= n_words) break;
        const uint32_t count = word_info[w] & 127u;
        if (lane >= count) continue;  // padding lanes of a layer's last word
        const size_t j = (size_t)w * 64u + lane;
        float s = bf16_bits_to_f32(gv[e][0]);
#pragma unroll
        for (int i = 1; i < WMAX; ++i) {
            if (i >= W) break;
            s = s + bf16_bits_to_f32(gv[e][i]);
        }
        const float gbar = s / (float)W;
        const float mn = sc.beta1 * mo[e] + sc.c1 * gbar;
        const float vv = sc.beta2 * (mo[e] * mo[e]) + sc.c2 * (gbar * gbar);
        float u = mn / (sqrtf(vv) + sc.eps);
        if (sc.wd != 0.0f) u = u + sc.wd * xo[e];
        __builtin_nontemporal_store(vv, &v[j]);
        __builtin_nontemporal_store(mn, &m[j]);
        __builtin_nontemporal_store(xo[e] - sc.lr * u, &x[j]);
    }
}

hipError_t launch_dense_adams(hipStream_t s, const uint16_t* word_info, uint32_t n_words, const WorkerPtrs& wp,
                              const StepScalars& sc, float* x, float* m, float* v) {
    if (n_words == 0) return hipSuccess;
#define SCAPE_DENSE_CASE(WV)                                                                                \
    case WV:                                                                                                \
        hipLaunchKernelGGL(k_dense_adams<WV>,                                                               \
                           dim3((n_words + kWaves * da_words<WV>() - 1) / (kWaves * da_words<WV>())),       \
                           dim3(kBlock), 0, s, word_info, n_words, wp, sc, x, m, v);                        \
        break;
    switch (sc.W) {
        SCAPE_DENSE_CASE(1)
        SCAPE_DENSE_CASE(2)
        SCAPE_DENSE_CASE(3)
        SCAPE_DENSE_CASE(4)
        SCAPE_DENSE_CASE(8)
        SCAPE_DENSE_CASE(16)
        SCAPE_DENSE_CASE(32)
        default:
            hipLaunchKernelGGL(k_dense_adams<0>, dim3((n_words + kWaves - 1) / kWaves), dim3(kBlock), 0, s, word_info,
                               n_words, wp, sc, x, m, v);
    }
#undef SCAPE_DENSE_CASE
    return hipGetLastError();
}

// Sparse pass: positions q of the current mask, kUpdatePer per thread (strided
// by the workgroup size so that idx, the sparse buffers and the m stash are
// read contiguously), every load issued before the arithmetic.  The pass runs
// beside the mask selection's record passes on another stream; its grid is
// capped at two workgroups per CU, striding over the positions (measured on
// the 0.35B, 0.55B and 1.75B workloads: 512 and no cap were equally fast,
// 256 and 128 starved the pass where it is long, W = 8 at keep 1/10).
#ifndef SCAPE_UPDATE_PER
#define SCAPE_UPDATE_PER 8  // with few workgroups, more positions in flight per thread
#endif
#ifndef SCAPE_UPDATE_GRID
#define SCAPE_UPDATE_GRID 512
#endif

constexpr int kUpdatePer = SCAPE_UPDATE_PER;

constexpr uint32_t kUpdateGrid = SCAPE_UPDATE_GRID;  // workgroups at most (0: one per chunk)

// With XV the parameters and the second moment are one array of (x, v)
// pairs, 8 bytes per element: the pass gathers and stores a position's pair
// with one access each instead of touching two arrays (measured on 17.5M
// positions at 1% density: 1.4-1.7 ms against 2.1-2.5 ms with x and v apart).
template <int WT, bool XV>
__global__ __launch_bounds__(kBlock) void k_reduce_update(WorkerPtrs wp, StepScalars sc, float* __restrict__ x,
                                                          float* __restrict__ m, float* __restrict__ v,
                                                          const uint32_t* __restrict__ idx,
                                                          const uint32_t* __restrict__ prefix,
                                                          const float* __restrict__ m_stash, uint32_t n_words,
                                                          uint32_t n_pad, uint32_t k_cap) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    constexpr int WMAX = WT > 0 ? WT : SCAPE_MAX_WORKERS;
    const uint32_t total = prefix[n_words];
    const uint32_t cnt = total < k_cap ? total : k_cap;
    const int W = WT > 0 ? WT : sc.W;
    const float fW = (float)W;
    f32x2* __restrict__ xv = reinterpret_cast<f32x2*>(x);
    constexpr uint32_t chunk = kBlock * kUpdatePer;
    for (uint32_t base = blockIdx.x * chunk; base < cnt; base += gridDim.x * chunk) {
    const uint32_t q0 = base + threadIdx.x;
    // Every load is unconditional, at a position clamped into [0, cnt) and an
    // element index clamped into [0, n_pad) (idx, the m stash and the sparse
    // buffers hold k_cap >= cnt entries, x holds n_pad): a guarded load
    // compiles to a branch and a wait for all outstanding loads, which
    // serialized the positions.  Only the stores are guarded.
    uint32_t qc[kUpdatePer], jj[kUpdatePer];
    float mo[kUpdatePer], xv0[kUpdatePer], s[kUpdatePer];
    bool ok[kUpdatePer];
#pragma unroll
    for (int u = 0; u < kUpdatePer; ++u) {
        const uint32_t q = q0 + u * kBlock;
        qc[u] = q < cnt ? q : cnt - 1u;
        jj[u] = idx[qc[u]];
        ok[u] = q < cnt && jj[u] < n_pad;
    }
#pragma unroll
    for (int u = 0; u < kUpdatePer; ++u) {
        mo[u] = m_stash[qc[u]];
        const uint32_t jc = jj[u] < n_pad ? jj[u] : 0u;
        // cached: the store below merges into the line in L2
        xv0[u] = XV ? xv[jc].x : x[jc];
        s[u] = wp.b[0][qc[u]];
    }
#pragma unroll
    for (int i = 1; i < WMAX; ++i) {
        if (i >= W) break;
#pragma unroll
        for (int u = 0; u < kUpdatePer; ++u) s[u] = s[u] + wp.b[i][qc[u]];
    }
#pragma unroll
    for (int u = 0; u < kUpdatePer; ++u) {
        if (!ok[u]) continue;
        const float bb = s[u] / fW;
        const float ghat = (bb - sc.beta1 * mo[u]) / sc.c1;
        const float vv = sc.beta2 * (mo[u] * mo[u]) + sc.c2 * (ghat * ghat);
        float upd = bb / (sqrtf(vv) + sc.eps);
        if (sc.wd != 0.0f) upd = upd + sc.wd * xv0[u];
        // m (and v when apart) are stored non-temporally; x, or the (x, v)
        // pair, goes through L2, where its line is already held by the gather
        // (both measured faster)
        __builtin_nontemporal_store(bb, &m[jj[u]]);
        if (XV) {
            f32x2 p;
            p.x = xv0[u] - sc.lr * upd;
            p.y = vv;
            xv[jj[u]] = p;
        } else {
            __builtin_nontemporal_store(vv, &v[jj[u]]);
            x[jj[u]] = xv0[u] - sc.lr * upd;
        }
    }
    }
}

hipError_t launch_reduce_update(hipStream_t s, const WorkerPtrs& wp, const StepScalars& sc, float* x, float* m,
                                float* v, bool xv_pairs, const uint32_t* cur_idx, const uint32_t* cur_prefix,
                                const float* m_stash, uint32_t n_words, uint32_t n_pad, uint32_t k_cap) {
    if (k_cap == 0) return hipSuccess;
    uint32_t blocks = (k_cap + kBlock * kUpdatePer - 1) / (kBlock * kUpdatePer);
    if (kUpdateGrid > 0 && blocks > kUpdateGrid) blocks = kUpdateGrid;
    const dim3 grid(blocks);
#define SCAPE_RU_LAUNCH(WV, XVV)                                                                                \
    hipLaunchKernelGGL((k_reduce_update<WV, XVV>), grid, dim3(kBlock), 0, s, wp, sc, x, m, v, cur_idx, cur_prefix, \
                       m_stash, n_words, n_pad, k_cap)
#define SCAPE_RU_CASE(WV)                        \
    case WV:                                     \
        if (xv_pairs) SCAPE_RU_LAUNCH(WV, true); \
        else SCAPE_RU_LAUNCH(WV, false);         \
        break;
    switch (sc.W) {
        SCAPE_RU_CASE(1)
        SCAPE_RU_CASE(2)
        SCAPE_RU_CASE(3)
        SCAPE_RU_CASE(4)
        SCAPE_RU_CASE(8)
        SCAPE_RU_CASE(16)
        SCAPE_RU_CASE(32)
        default:
            if (xv_pairs) SCAPE_RU_LAUNCH(0, true);
            else SCAPE_RU_LAUNCH(0, false);
    }
#undef SCAPE_RU_LAUNCH
#undef SCAPE_RU_CASE
    return hipGetLastError();
}

// Statistic keys from a given m-tilde (the standalone mask build): a wave
// handles kKeyWords consecutive words, one-shot and in the dense pass's
// XCD-aware order.  All of the wave's loads (m-tilde non-temporally, and the
// words' descriptors) are issued before any key is formed, at words clamped
// into the range, so that enough bytes are in flight per wave: with one 256-byte
// word per wave the pass ran at about 2.2 TB/s.  m-tilde holds n_pad
// elements, so every lane may load; the padding lanes of a layer's last word
// store nothing.
constexpr uint32_t kKeyWords = 8;

__global__ __launch_bounds__(kEfBlock) void k_keys_from_mtilde(const uint16_t* __restrict__ word_info,
                                                               uint32_t w_begin, uint32_t w_end,
                                                               const float* __restrict__ mtilde,
                                                               uint16_t* __restrict__ key16) {
    const uint32_t blk = kEfXcd ? xcd_block(blockIdx.x, gridDim.x) : blockIdx.x;
    const uint32_t w0 = w_begin + (blk * kEfWaves + threadIdx.x / 64) * kKeyWords;
    if (w0 >= w_end) return;
    const uint32_t lane = lane_id();
    float mt[kKeyWords];
    uint32_t info[kKeyWords];
#pragma unroll
    for (uint32_t e = 0; e < kKeyWords; ++e) {
        const uint32_t w = min(w0 + e, w_end - 1u);
        mt[e] = stream_load(&mtilde[(size_t)w * 64u + lane]);
        info[e] = word_info[w];
    }
#pragma unroll
    for (uint32_t e = 0; e < kKeyWords; ++e) {
        if (w0 + e < w_end && lane < (info[e] & 127u))
            key16[(size_t)(w0 + e) * 64u + lane] = (uint16_t)(magnitude_key(mt[e]) >> kKeyShift);
    }
}

hipError_t launch_keys_from_mtilde(hipStream_t s, const uint16_t* word_info, uint32_t w_begin, uint32_t w_end,
                                   const float* mtilde, uint16_t* key16) {
    if (w_end <= w_begin) return hipSuccess;
    const uint32_t per_block = kEfWaves * kKeyWords;
    hipLaunchKernelGGL(k_keys_from_mtilde, dim3((w_end - w_begin + per_block - 1) / per_block), dim3(kEfBlock), 0, s,
                       word_info, w_begin, w_end, mtilde, key16);
    return hipGetLastError();
}

struct BufPtrs {
    const float* b[SCAPE_MAX_WORKERS];
};

// The W-way mean on its own: the W loads of a position are issued together
// (W fixed at compile time for the common counts), then summed in worker order.
template <int WT>
__global__ __launch_bounds__(kBlock) void k_reduce_sparse(BufPtrs bp, int32_t w_rt, uint64_t k, float* __restrict__ out) {
    constexpr int WMAX = WT > 0 ? WT : SCAPE_MAX_WORKERS;
    const int W = WT > 0 ? WT : w_rt;
    const float fW = (float)W;
    for (uint64_t q = (uint64_t)blockIdx.x * kBlock + threadIdx.x; q < k; q += (uint64_t)gridDim.x * kBlock) {
        float v[WMAX];
#pragma unroll
        for (int i = 0; i < WMAX; ++i) {
            if (i >= W) break;
            v[i] = bp.b[i][q];
        }
        float s = v[0];
#pragma unroll
        for (int i = 1; i < WMAX; ++i) {
            if (i >= W) break;
            s = s + v[i];
        }
        out[q] = s / fW;
    }
}

hipError_t launch_reduce_sparse(hipStream_t s, const float* const* bufs, int32_t W, int64_t k, float* out) {
    if (k <= 0) return hipSuccess;
    BufPtrs bp{};
    for (int i = 0; i < W; ++i) bp.b[i] = bufs[i];
    uint64_t blocks = ((uint64_t)k + kBlock - 1) / kBlock;
    if (blocks > 16384u) blocks = 16384u;
    const dim3 grid((uint32_t)blocks);
#define SCAPE_RS_CASE(WV)                                                                                 \
    case WV:                                                                                              \
        hipLaunchKernelGGL(k_reduce_sparse<WV>, grid, dim3(kBlock), 0, s, bp, W, (uint64_t)k, out); \
        break;
    switch (W) {
        SCAPE_RS_CASE(1)
        SCAPE_RS_CASE(2)
        SCAPE_RS_CASE(3)
        SCAPE_RS_CASE(4)
        SCAPE_RS_CASE(8)
        SCAPE_RS_CASE(16)
        SCAPE_RS_CASE(32)
        default:
            hipLaunchKernelGGL(k_reduce_sparse<0>, grid, dim3(kBlock), 0, s, bp, W, (uint64_t)k, out);
    }
#undef SCAPE_RS_CASE
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

// Several ranges zeroed by one launch: row y of the grid takes range y.
__global__ __launch_bounds__(kBlock) void k_zero_ranges(ZeroRanges zr) {
    uint32_t* __restrict__ p = zr.p[blockIdx.y];
    const uint64_t n = zr.n[blockIdx.y];
    for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (uint64_t)gridDim.x * kBlock) p[i] = 0u;
}

hipError_t launch_zero_ranges(hipStream_t s, const ZeroRanges& zr) {
    uint64_t most = 0;
    for (int i = 0; i < zr.count; ++i) most = zr.n[i] > most ? zr.n[i] : most;
    if (most == 0) return hipSuccess;
    uint64_t blocks = (most + kBlock - 1) / kBlock;
    if (blocks > 8192u) blocks = 8192u;
    hipLaunchKernelGGL(k_zero_ranges, dim3((uint32_t)blocks, (uint32_t)zr.count), dim3(kBlock), 0, s, zr);
    return hipGetLastError();
}

}  // namespace scape
