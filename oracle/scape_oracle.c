/*
 * scape_oracle.c - the oracle of the SCAPE per-worker optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this file's library.  The product
 * path never does, and shares no code with it.
 *
 * A plain, slow, scalar C implementation of what one SCAPE step computes,
 * written step by step from the pages.  The pages:
 *   [abs]  "SCAPE: Accurate and Efficient LLM Training with Extreme Sparse
 *          Communication", shd-paper.top page, English abstract.
 *   [TS-n] gist.science "Technical Summary: SCAPE - Accurate and Efficient
 *          LLM Training with Extreme Sparse Communication", section n
 *          (2 = Methodology, with the headings "Key Design Insights",
 *          "Partitioned Mask Synchronization", "Delayed Mask Usage (One-Step
 *          Lag)", "Single-Buffer Second-Moment Reconstruction", "Memory
 *          Optimization").
 * The pages print no formula.  Where they leave a step open, this file takes
 * one explicit reading; each reading is named at the code that uses it:
 *   R-normaliser  v = beta2*m_prev^2 + (1-beta2)*g_hat^2 (AdamS's
 *                 momentum-and-gradient denominator), no bias correction,
 *                 eps outside the square root, decoupled weight decay.
 *   R-statistic   the mask statistic of a layer is its owner worker's local
 *                 error-compensated first-moment candidate.
 *   R-owner       a layer is owned by the shard holding its midpoint under an
 *                 even split of the flat buffer into P shards.
 *   R-buffer      the sparse buffer carries the workers' first-moment
 *                 candidates at the masked positions, in ascending position
 *                 order (values only; the mask is global).
 *   R-mean        the all-reduce is a mean: a sum over workers in order
 *                 0..W-1, then a division by W.
 *   R-offmask     off-mask x, m and v are unchanged; only residuals grow.
 *   R-k           k = ceil(n * keep_num / keep_den); ties go to the lower
 *                 position; keys are the bit patterns of |candidate|.
 *   R-layout      tensors are concatenated, each starting on a 64-element
 *                 boundary; mask bits are LSB-first in 64-bit words.
 *   R-fillin      the "fill-in" alternative to partitioned masks: every
 *                 worker ranks every layer on its own first-moment candidate
 *                 (the same per-layer top-k and tie rule as R-k) and the
 *                 global mask is the union of the workers' masks.
 *   R-dense       the dense AdamS step the pages compare against is plain
 *                 data parallelism: the workers' gradients are averaged
 *                 (sum in order 0..W-1, then division by W) on every element
 *                 and that average drives the same AdamS update as
 *                 R-normaliser, with no residual and no mask.
 *
 * Threads: built with OpenMP, the loops run in parallel over layers (each
 * layer's elements in order, its first compaction slot counted beforehand)
 * and over positions of the sparse buffers.  Every iteration writes its own
 * outputs and no floating-point sum is split across threads, so the results
 * do not depend on the thread count.
 *
 * Precision: every floating-point value is fp32, every operation rounds to
 * nearest even, and nothing is contracted into a fused multiply-add (the file
 * is compiled with -ffp-contract=off, no fast-math).  fp32 is the state
 * precision of the workloads, and the mask is an integer decision taken on
 * fp32 statistics, so the oracle takes it in that same precision.
 *
 * Parity pins (tests/test_oracle_pins.py) tie each function to something
 * outside itself: brute-force ranking, library packbits/cumsum, exact dyadic
 * arithmetic, a dense fp64 average, a dense fp64 AdamS, power-of-two scaling;
 * the dense step by a hand-worked dyadic example, by agreement with the
 * SCAPE step under a full mask, and by exact scaling and sign symmetries;
 * the fill-in union by a brute-force ranking in the tests, by its bounds
 * (k to W*k set bits per layer), monotonicity in W and disjoint supports.
 * The AdamS normaliser form itself (R-normaliser) is a reading the pages do
 * not fix: parity unpinned for that form beyond its algebraic special cases.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the parallel loops use. */
int oracle_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* Layout, kept counts, ownership                                           */
/* ------------------------------------------------------------------------ */

/* R-k: kept count of a layer of n elements at keep = num/den, rounded up. */
int64_t oracle_keep_count(int64_t n, uint32_t num, uint32_t den) {
    unsigned __int128 p = (unsigned __int128)(uint64_t)n * num;
    return (int64_t)((p + den - 1) / den);
}

/* R-owner: shard whose interval [s*N/P, (s+1)*N/P) holds the layer midpoint
 * off + n/2 (Partitioned Mask Synchronization, TS-2: masks are built per
 * worker, for its partitioned layers, aligned with optimizer sharding). */
int32_t oracle_owner(int64_t off, int64_t n, int64_t n_total, int32_t P) {
    if (n_total <= 0) return 0;
    int64_t s = (int64_t)(((__int128)P * (2 * off + n)) / (2 * (__int128)n_total));
    if (s > P - 1) s = P - 1;
    return (int32_t)s;
}

/* R-layout: each tensor starts on a 64-element boundary. */
void oracle_layout(int32_t L, const int64_t* n, uint32_t keep_num, uint32_t keep_den, int32_t P,
                   int64_t* off, int64_t* k, int32_t* owner, int64_t* n_pad) {
    int64_t cur = 0;
    for (int32_t l = 0; l < L; ++l) {
        off[l] = cur;
        cur += (n[l] + 63) / 64 * 64;
        k[l] = oracle_keep_count(n[l], keep_num, keep_den);
    }
    *n_pad = cur;
    for (int32_t l = 0; l < L; ++l) owner[l] = oracle_owner(off[l], n[l], cur, P);
}

/* ------------------------------------------------------------------------ */
/* 1-bit masks (Memory Optimization, TS-2: packed single-bit mask format)    */
/* ------------------------------------------------------------------------ */

/* Element j is bit (j mod 64) of word j/64; bits past n are zero. */
void oracle_pack(const uint8_t* pred, int64_t n, uint64_t* words) {
    int64_t nw = (n + 63) / 64;
    for (int64_t w = 0; w < nw; ++w) words[w] = 0;
    for (int64_t j = 0; j < n; ++j)
        if (pred[j]) words[j / 64] |= (uint64_t)1 << (j % 64);
}

void oracle_unpack(const uint64_t* words, int64_t n, uint8_t* pred) {
    for (int64_t j = 0; j < n; ++j) pred[j] = (uint8_t)((words[j / 64] >> (j % 64)) & 1u);
}

static int bit_at(const uint64_t* words, int64_t j) { return (int)((words[j / 64] >> (j % 64)) & 1u); }

/* Positions of the set bits in ascending order, and prefix[w] = number of set
 * bits in words 0..w-1 (n_words+1 entries).  Returns the count; positions past
 * idx_cap are counted but not stored. */
int64_t oracle_mask_index(const uint64_t* words, int64_t n_words, uint32_t* idx, int64_t idx_cap,
                          uint32_t* prefix) {
    int64_t c = 0;
    for (int64_t w = 0; w < n_words; ++w) {
        if (prefix) prefix[w] = (uint32_t)c;
        for (int b = 0; b < 64; ++b) {
            if ((words[w] >> b) & 1u) {
                if (idx && c < idx_cap) idx[c] = (uint32_t)(w * 64 + b);
                ++c;
            }
        }
    }
    if (prefix) prefix[n_words] = (uint32_t)c;
    return c;
}

/* ------------------------------------------------------------------------ */
/* Top-k mask from first-moment statistics                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
    uint32_t key;
    uint32_t pos;
} keyed_pos;

/* Total order: larger key first, then lower position first (R-k). */
static int by_key_desc_pos_asc(const void* a, const void* b) {
    const keyed_pos* x = (const keyed_pos*)a;
    const keyed_pos* y = (const keyed_pos*)b;
    if (x->key != y->key) return x->key > y->key ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

/* sel[j] = 1 for the k elements of key[0..n) that come first in the order. */
void oracle_topk(const uint32_t* key, int64_t n, int64_t k, uint8_t* sel) {
    keyed_pos* a = (keyed_pos*)malloc(sizeof(keyed_pos) * (size_t)(n > 0 ? n : 1));
    for (int64_t j = 0; j < n; ++j) {
        a[j].key = key[j];
        a[j].pos = (uint32_t)j;
        sel[j] = 0;
    }
    qsort(a, (size_t)n, sizeof(keyed_pos), by_key_desc_pos_asc);
    for (int64_t q = 0; q < k && q < n; ++q) sel[a[q].pos] = 1;
    free(a);
}

/* Mask key of a first-moment value: bit pattern of its magnitude. */
static uint32_t magnitude_key(float v) {
    float a = fabsf(v);
    uint32_t u;
    memcpy(&u, &a, 4);
    return u;
}

/* Per-layer top-k over flat keys (layers as in oracle_layout), written into
 * the words that cover each layer.  Only layers with owner == shard are built
 * when shard >= 0; other words are left untouched. */
void oracle_mask_from_keys(int32_t L, const int64_t* off, const int64_t* n, const int64_t* k,
                           const int32_t* owner, int32_t shard, const uint32_t* key, uint64_t* words) {
    /* layers own disjoint words (each starts on a 64-element boundary) */
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t l = 0; l < L; ++l) {
        if (shard >= 0 && owner[l] != shard) continue;
        uint8_t* sel = (uint8_t*)malloc((size_t)(n[l] > 0 ? n[l] : 1));
        oracle_topk(key + off[l], n[l], k[l], sel);
        int64_t w0 = off[l] / 64, w1 = (off[l] + n[l] + 63) / 64;
        for (int64_t w = w0; w < w1; ++w) words[w] = 0;
        for (int64_t j = 0; j < n[l]; ++j)
            if (sel[j]) words[(off[l] + j) / 64] |= (uint64_t)1 << ((off[l] + j) % 64);
        free(sel);
    }
}

/* The fill-in union (R-fillin): worker i's per-layer top-k of its own keys
 * keys[i] over every layer, OR-ed into words (the caller zeroes words first).
 * This is what Partitioned Mask Synchronization (TS-2) avoids: when every
 * worker builds a mask for every layer, the union fills in as W grows. */
void oracle_union_mask(int32_t L, const int64_t* off, const int64_t* n, const int64_t* k, int32_t W,
                       const uint32_t* const* keys, uint64_t* words) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t l = 0; l < L; ++l) {
        for (int32_t i = 0; i < W; ++i) {
            uint8_t* sel = (uint8_t*)malloc((size_t)(n[l] > 0 ? n[l] : 1));
            oracle_topk(keys[i] + off[l], n[l], k[l], sel);
            for (int64_t j = 0; j < n[l]; ++j)
                if (sel[j]) words[(off[l] + j) / 64] |= (uint64_t)1 << ((off[l] + j) % 64);
            free(sel);
        }
    }
}

/* Keys of an m-tilde array (for the standalone mask build). */
void oracle_keys_of(const float* mtilde, int64_t n, uint32_t* key) {
    for (int64_t j = 0; j < n; ++j) key[j] = magnitude_key(mtilde[j]);
}

/* ------------------------------------------------------------------------ */
/* Reduction of the workers' sparse buffers                                 */
/* ------------------------------------------------------------------------ */

/* R-mean (Single-Buffer Second-Moment Reconstruction, TS-2: one synchronized
 * sparse buffer b-bar).  out[q] = ((b_0[q] + b_1[q]) + ... + b_{W-1}[q]) / W. */
void oracle_reduce(const float* const* bufs, int32_t W, int64_t k, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < k; ++q) {
        float s = bufs[0][q];
        for (int32_t i = 1; i < W; ++i) s = s + bufs[i][q];
        out[q] = s / (float)W;
    }
}

static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* One optimizer step                                                       */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t L;
    const int64_t* off;    /* flat offset of each layer (multiple of 64) */
    const int64_t* n;      /* elements of each layer */
    const int64_t* k;      /* kept count of each layer */
    const int32_t* owner;  /* worker whose candidate ranks the layer */
    int64_t n_pad;         /* flat length, multiple of 64 */
    int32_t W;
    float beta1, beta2, lr, eps, weight_decay;
} oracle_problem;

/*
 * One step t.  Inputs: state x, m, v, residuals r[i]; bf16 gradients g[i];
 * the mask M_t as words (cur_words).  Outputs, all caller-allocated:
 *   sent[i][0..cnt)  worker i's sparse buffer (candidates at M_t, ascending),
 *   bbar[0..cnt)     the reduced buffer,
 *   key[n_pad]       mask statistic per element (0 in padding),
 *   next_words, next_idx (sum k entries), next_prefix (n_words+1): M_{t+1}.
 * sent_cap bounds the buffers; returns cnt = |M_t| or -1 if it exceeds sent_cap.
 */
int64_t oracle_step(const oracle_problem* P, float* x, float* m, float* v, float* const* r,
                    const uint16_t* const* g, const uint64_t* cur_words, float* const* sent,
                    float* bbar, int64_t sent_cap, uint32_t* key, uint64_t* next_words,
                    uint32_t* next_idx, uint32_t* next_prefix) {
    const float b1 = P->beta1, b2 = P->beta2;
    const float c1 = 1.0f - b1; /* (1 - beta1) */
    const float c2 = 1.0f - b2; /* (1 - beta2) */
    const int32_t W = P->W;
    const int64_t n_words = P->n_pad / 64;

    /* Positions of M_t in ascending order. */
    int64_t cnt = oracle_mask_index(cur_words, n_words, NULL, 0, NULL);
    if (cnt > sent_cap) return -1;
    uint32_t* pos = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(cnt > 0 ? cnt : 1));
    oracle_mask_index(cur_words, n_words, pos, cnt, NULL);

    for (int64_t j = 0; j < P->n_pad; ++j) key[j] = 0;

    /* (1) Error feedback: each worker adds its gradient to its residual, a_i =
     *     r_i + g_i (Problem Statement, TS-1, and Key Design Insights, TS-2:
     *     error feedback with residuals).  (2) AdamS first-moment candidate
     *     m~_i = beta1*m + (1-beta1)*a_i, from the error-compensated gradient
     *     ([abs]: masks come from first-moment statistics, not raw
     *     gradients).  (3) Compaction: at the positions of M_t the candidates
     *     go into the worker's sparse buffer and the residual is cleared; off
     *     the mask the residual keeps a_i (R-buffer).  The owner's candidate
     *     gives the mask statistic (R-statistic). */
    /* The layers are cut into runs of at most 2^20 elements, and the first
     * compaction slot of each run (the masked positions before it) is
     * counted beforehand, so that the runs can be processed independently;
     * inside a run, elements go in order. */
    const int64_t run_len = (int64_t)1 << 20;
    int64_t n_runs = 0;
    for (int32_t l = 0; l < P->L; ++l) n_runs += (P->n[l] + run_len - 1) / run_len;
    int64_t* run_j0 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_runs > 0 ? n_runs : 1));
    int64_t* run_j1 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_runs > 0 ? n_runs : 1));
    int32_t* run_l = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_runs > 0 ? n_runs : 1));
    int64_t* q0 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_runs > 0 ? n_runs : 1));
    {
        int64_t r = 0, c = 0;
        for (int32_t l = 0; l < P->L; ++l) {
            for (int64_t e0 = 0; e0 < P->n[l]; e0 += run_len, ++r) {
                const int64_t e1 = e0 + run_len < P->n[l] ? e0 + run_len : P->n[l];
                run_l[r] = l;
                run_j0[r] = P->off[l] + e0;
                run_j1[r] = P->off[l] + e1;
                q0[r] = c;
                for (int64_t j = run_j0[r]; j < run_j1[r]; ++j) c += bit_at(cur_words, j);
            }
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t rr = 0; rr < n_runs; ++rr) {
        const int32_t l = run_l[rr];
        int64_t q = q0[rr];
        for (int64_t j = run_j0[rr]; j < run_j1[rr]; ++j) {
            const float mo = m[j];
            const float bm = b1 * mo;
            const int masked = bit_at(cur_words, j);
            for (int32_t i = 0; i < W; ++i) {
                const float a = r[i][j] + bf16_to_f32(g[i][j]);
                const float mt = bm + c1 * a;
                if (i == P->owner[l]) key[j] = magnitude_key(mt);
                if (masked) {
                    sent[i][q] = mt;
                    r[i][j] = 0.0f;
                } else {
                    r[i][j] = a;
                }
            }
            if (masked) ++q;
        }
    }

    free(q0);
    free(run_j0);
    free(run_j1);
    free(run_l);

    /* (4) The single synchronized sparse buffer: mean over workers (R-mean). */
    oracle_reduce((const float* const*)sent, W, cnt, bbar);

    /* (5) Single-Buffer Second-Moment Reconstruction (TS-2): from b-bar alone,
     *     g_hat = (b-bar - beta1*m_prev)/(1-beta1) is the workers' averaged
     *     error-compensated gradient; then the AdamS normaliser
     *     (R-normaliser), m = b-bar, and the parameter update.  Off-mask
     *     coordinates are untouched (R-offmask). */
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < cnt; ++s) {
        const int64_t j = pos[s];
        const float mo = m[j];
        const float bb = bbar[s];
        const float ghat = (bb - b1 * mo) / c1;
        v[j] = b2 * (mo * mo) + c2 * (ghat * ghat);
        m[j] = bb;
        float u = bb / (sqrtf(v[j]) + P->eps);
        if (P->weight_decay != 0.0f) u = u + P->weight_decay * x[j];
        x[j] = x[j] - P->lr * u;
    }

    /* (6) Mask for step t+1: per layer, the k largest statistics, built by
     *     the layer's owner (Partitioned Mask Synchronization, TS-2), packed
     *     to bits; it is applied at the next step (Delayed Mask Usage, TS-2). */
    for (int64_t w = 0; w < n_words; ++w) next_words[w] = 0;
    oracle_mask_from_keys(P->L, P->off, P->n, P->k, P->owner, -1, key, next_words);
    int64_t ktot = 0;
    for (int32_t l = 0; l < P->L; ++l) ktot += P->k[l] < P->n[l] ? P->k[l] : P->n[l];
    oracle_mask_index(next_words, n_words, next_idx, ktot, next_prefix);

    free(pos);
    return cnt;
}

/* ------------------------------------------------------------------------ */
/* The dense AdamS step (the comparison baseline)                           */
/* ------------------------------------------------------------------------ */

/*
 * One dense AdamS step on W simulated workers: the baseline the pages measure
 * SCAPE against ([abs]: per-step speedup over dense AdamS; TS Results, Per-Step
 * Speedup).  Reading R-dense: on every element of every layer the workers'
 * bf16 gradients are averaged in worker order, and the average drives the
 * AdamS update of R-normaliser.  Padding elements are not touched.
 */
void oracle_dense_step(const oracle_problem* P, float* x, float* m, float* v, const uint16_t* const* g) {
    const float b1 = P->beta1, b2 = P->beta2;
    const float c1 = 1.0f - b1;
    const float c2 = 1.0f - b2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t l = 0; l < P->L; ++l) {
        for (int64_t e = 0; e < P->n[l]; ++e) {
            const int64_t j = P->off[l] + e;
            /* the dense all-reduce of the gradients, as a mean (R-dense) */
            float s = bf16_to_f32(g[0][j]);
            for (int32_t i = 1; i < P->W; ++i) s = s + bf16_to_f32(g[i][j]);
            const float gbar = s / (float)P->W;
            /* AdamS: the new first moment, the normaliser from the previous
             * first moment and the gradient, then the parameter update */
            const float mo = m[j];
            const float mn = b1 * mo + c1 * gbar;
            v[j] = b2 * (mo * mo) + c2 * (gbar * gbar);
            m[j] = mn;
            float u = mn / (sqrtf(v[j]) + P->eps);
            if (P->weight_decay != 0.0f) u = u + P->weight_decay * x[j];
            x[j] = x[j] - P->lr * u;
        }
    }
}
