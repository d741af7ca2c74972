/*
 * scape.h - C ABI of libscape, the SCAPE per-worker optimizer step on
 * AMD Instinct MI355X (gfx950).
 *
 * SCAPE is the sparse-communication distributed optimizer of "SCAPE: Accurate
 * and Efficient LLM Training with Extreme Sparse Communication" (Zheng, Chen,
 * Xie, Zhang; arXiv 2607.01678).  Citations below name the page and section:
 *   [abs]   shd-paper.top page, English abstract;
 *   [TS-n]  gist.science "Technical Summary: SCAPE - Accurate and Efficient
 *           LLM Training with Extreme Sparse Communication", section n.
 * The pages print no formula; where they leave a step open the library takes
 * one explicit reading, stated at the entry point that uses it.
 *
 * Conventions for every entry point:
 *   - Return value: SCAPE_OK (0) or a negative SCAPE_ERR_* code.  Nothing
 *     throws.  scape_last_error() gives a text for the calling thread's last
 *     failure.  Arguments are validated on the host before anything is
 *     enqueued; on a validation error nothing is launched and no output is
 *     touched.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Device work is
 *     enqueued asynchronously on it; no call synchronizes the host, except
 *     scape_init/scape_destroy/scape_profile_read as noted.
 *   - Pointers named "device" point to device memory the caller owns; they
 *     must be 16-byte aligned unless stated otherwise.  Pointer arrays
 *     (`r`, `g`, `sparse_bufs`) are host arrays of W device pointers.
 *   - A context must not be used on two streams at once; separate contexts
 *     are independent.
 *
 * Layout (one flat buffer for all parameter tensors): tensor l starts at
 * element offset layer_offset[l], a multiple of 64, and the flat length n_pad
 * is a multiple of 64 (elements between tensors are padding and are never
 * read or written by the step).  A mask over the flat buffer is stored as
 *   bits[n_pad/64]           element j is bit (j % 64) of word j/64, LSB first;
 *   idx[k_total]             the set positions in ascending order (uint32);
 *   block_prefix[n_pad/64+1] number of set bits in words 0..w-1.
 * Masks use one bit per element, the packed single-bit format of the Memory
 * Optimization paragraph of [TS-2].
 */
#ifndef SCAPE_H
#define SCAPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SCAPE_VERSION_MAJOR 1
#define SCAPE_VERSION_MINOR 0

#define SCAPE_OK 0
#define SCAPE_ERR_INVALID_ARG (-1) /* null pointer, bad enum, out-of-range scalar     */
#define SCAPE_ERR_SHAPE (-2)       /* sizes that do not fit the layout or the limits  */
#define SCAPE_ERR_ALIGN (-3)       /* a device pointer is not aligned as required     */
#define SCAPE_ERR_OOM (-4)         /* device allocation failed or would exceed limits */
#define SCAPE_ERR_HIP (-5)         /* a HIP call failed; text in scape_last_error()   */
#define SCAPE_ERR_STATE (-6)       /* call not valid in the context's current state   */

#define SCAPE_MAX_WORKERS 32

typedef struct scape_ctx scape_ctx;

/* Problem description.  All fields are read at scape_init and copied. */
typedef struct scape_config {
    int32_t num_layers;         /* L >= 1 parameter tensors ("layers")               */
    const int64_t* layer_numel; /* host array [L], each >= 0, sum of padded sizes
                                   below 2^31 elements                               */
    int32_t workers;            /* W, 1..SCAPE_MAX_WORKERS simulated workers         */
    int32_t owner_shards;       /* P, 1..W ownership shards; 0 means W               */
    float beta1, beta2;         /* AdamS moment coefficients, each in [0, 1)         */
    float lr, eps, weight_decay;
    uint32_t keep_num, keep_den;/* kept fraction (1 - sparsity) = keep_num/keep_den,
                                   0 <= keep_num <= keep_den, keep_den >= 1          */
} scape_config;

/* A mask in the layout above; all three arrays are caller-owned device memory
 * (bits 8-byte aligned, idx and block_prefix 4-byte aligned). */
typedef struct scape_mask {
    uint64_t* bits;
    uint32_t* idx;
    uint32_t* block_prefix;
} scape_mask;

/* Library version. */
int scape_version(int32_t* major, int32_t* minor);

/* Text of the calling thread's last failure ("" if none).  The pointer stays
 * valid until the thread's next failing call. */
const char* scape_last_error(void);

/*
 * Host-only layout query (no GPU needed).  Kept count per layer:
 * k_l = ceil(n_l * keep_num / keep_den) (the pages evaluate 90% and 99%
 * sparsity, [abs]; rounding up keeps at least one element of a non-empty
 * layer).  Owner of layer l under P shards: the shard of an even split of
 * [0, n_pad) into P parts that holds the layer midpoint, capped at P-1 - the
 * layer-aligned ownership of Partitioned Mask Synchronization [TS-2].
 * Outputs may be NULL; layer_offset/layer_k/layer_owner have L entries.
 * Errors: INVALID_ARG / SHAPE for a config scape_init would reject.
 */
int scape_layout(const scape_config* cfg, int64_t* n_pad, int64_t* k_total, int64_t* layer_offset,
                 int64_t* layer_k, int32_t* layer_owner);

/* Host-only: owner shard of every layer for an arbitrary shard count P >= 1
 * (owner[L]).  Used to pick the layers of one worker's mask build. */
int scape_owner_map(const scape_config* cfg, int32_t num_shards, int32_t* owner);

/*
 * Create a context: validates the config, builds the layout and tile tables,
 * and allocates the context's own device workspaces (histograms, per-layer
 * selection state, candidate records, scan partials, statistic buffer) on the
 * current HIP device.  Synchronizes the device once (table upload).
 * Errors: INVALID_ARG, SHAPE, OOM, HIP.  *out is set only on success.
 */
int scape_init(const scape_config* cfg, scape_ctx** out);

/* Free a context and its workspaces (synchronizes the device).  NULL is OK. */
int scape_destroy(scape_ctx* ctx);

/* Device memory the context holds (its workspaces, in bytes), host only.
 * Grows by the offloaded step's buffers after its first call.
 * Errors: INVALID_ARG. */
int scape_workspace_bytes(const scape_ctx* ctx, int64_t* bytes);

/* Which exact fallbacks the context's last mask selection took (a
 * diagnostic; waits for the device): bit 0 = some layer's threshold fell
 * outside its sampled window or its window held more records than its
 * record space, and was redone from an exact histogram of its keys; bit 1 =
 * some layer's exact threshold bucket still did not fit its record space and
 * was decided by passes over its keys.  Either way the mask is the exact one.
 * Errors: INVALID_ARG, STATE, HIP. */
#define SCAPE_SELECT_EXACT_HISTOGRAM 1u
#define SCAPE_SELECT_KEY_PASSES 2u
int scape_selection_flags(scape_ctx* ctx, uint32_t* flags);

/* How the context selects a mask (per-layer top-k; the mask is the same
 * either way).  SAMPLED: a sampled histogram windows each layer's threshold,
 * one pass over the keys marks what lies above the window and records what
 * lies in it, and multi-workgroup passes over the records resolve the
 * remaining digits (about 20 launches; built for large layers).  COMPACT: an
 * exact histogram pass, then one pass that marks and records the threshold
 * bucket, whose records one workgroup per layer resolves (2 launches; built
 * for layers of up to a few million elements, where launches dominate).
 * AUTO (the default): COMPACT for a layer range whose layers all have at
 * most 2^22 elements, else SAMPLED.  Host only, takes effect from the next
 * call.  Errors: INVALID_ARG. */
#define SCAPE_SELECT_PATH_AUTO 0
#define SCAPE_SELECT_PATH_SAMPLED 1
#define SCAPE_SELECT_PATH_COMPACT 2
int scape_set_select_path(scape_ctx* ctx, int32_t path);

/* Where scape_step reduces and applies the update (the results are the same
 * either way).  on = 1 (the default): where the residuals are on the device,
 * the dense pass does it at the mask's positions (it holds every worker's
 * candidate of an element), so no separate update pass runs and the
 * selection follows the dense pass alone.  Where the mask keeps at most 1/32
 * of the elements the pass touches x, v and m at the masked elements only;
 * on denser masks it streams them whole and stores the other elements' old
 * values back.  Measured in a fresh GPU's first process: the 1.75B workload
 * (keep 1/100) 15.75-15.78 ms against 16.22-16.25 ms with the update as a
 * pass of its own, the GPT-345M-shaped one (keep 1/10) 7.58 against 7.92 ms.
 * on = 0: the update is a pass of its own, beside the selection.  Host only,
 * takes effect from the next call.  Errors: INVALID_ARG. */
int scape_set_update_in_dense_pass(scape_ctx* ctx, int32_t on);

/* How scape_step_offload moves the residuals (the results are the same
 * either way).  SCAPE_OFFLOAD_PATH_AUTO (the default): where every r_host[i]
 * lies in pinned host memory mapped for the GPU (hipHostMalloc, a pinned
 * torch tensor), the dense pass reads and writes them over PCIe itself, its
 * reads and writes in flight together; otherwise through the staging slots.
 * SCAPE_OFFLOAD_PATH_STAGED: always through the staging slots.  Host only,
 * takes effect from the next call.  Errors: INVALID_ARG. */
#define SCAPE_OFFLOAD_PATH_AUTO 0
#define SCAPE_OFFLOAD_PATH_STAGED 1
int scape_set_offload_path(scape_ctx* ctx, int32_t path);

/*
 * One SCAPE step on W simulated workers, all resident on this GPU.
 *
 * Per element j (in any tensor l, with mo = m[j] before the step):
 *   a_i  = r_i[j] + float(g_i[j])                 error feedback: the residual
 *                                                 keeps unsent gradient mass
 *                                                 ([TS-1] Problem Statement;
 *                                                 [TS-2] Key Design Insights)
 *   mt_i = beta1*mo + (1-beta1)*a_i               AdamS first-moment candidate
 *   r_i[j] = (j in M_t) ? 0 : a_i
 *   key[j] = bit pattern of |mt_owner(l)|         first-moment statistic of the
 *                                                 layer's owner ([abs])
 * At the positions of M_t (`cur`), in ascending order q = 0..|M_t|-1:
 *   sparse_bufs[i][q] = mt_i                      worker i's sparse buffer: the
 *                                                 payload one collective carries
 *   bbar = ((mt_0 + mt_1) + ... + mt_{W-1}) / W   the synchronized buffer
 *   g_hat = (bbar - beta1*mo) / (1-beta1)         averaged gradient and residual
 *                                                 recovered from bbar alone
 *                                                 ([TS-2] Single-Buffer Second-
 *                                                 Moment Reconstruction)
 *   v[j] = beta2*mo^2 + (1-beta2)*g_hat^2         AdamS normaliser (reading: no
 *                                                 bias correction)
 *   m[j] = bbar
 *   x[j] = x[j] - lr*(bbar/(sqrt(v[j]) + eps) + weight_decay*x[j])
 * Off M_t, x, m and v are unchanged.  Then M_{t+1} (`next`): per layer, the
 * k_l positions with the largest key, ties to the lower position ([TS-2]
 * Partitioned Mask Synchronization), written as bits, idx and block_prefix.
 * M_{t+1} is for the next call: the caller passes it as `cur` then ([TS-2]
 * Delayed Mask Usage).  The first step normally passes an all-zero mask.
 * Every floating-point operation is IEEE fp32, round to nearest even, in the
 * order written, with no fused multiply-add.
 *
 * Arguments (device, n_pad elements unless stated):
 *   x, m, v       fp32 state, updated in place;
 *   r[W]          fp32 residual of each worker, updated in place;
 *   g[W]          bfloat16 gradient bits (uint16) of each worker, read only;
 *   cur           M_t, read only, as written by scape_step/scape_mask_build/
 *                 scape_mask_index (bits, idx, block_prefix consistent);
 *                 positions beyond the first k_total set bits are treated as
 *                 unmasked;
 *   next          M_{t+1}, written; must not alias `cur`;
 *   sparse_bufs[W] fp32 device arrays of k_total entries, written (4-byte
 *                 alignment suffices);
 *   key_out       uint32 array (n_pad) for the full statistic keys, written
 *                 when not NULL (4 more bytes per element); may be NULL.  The
 *                 selection itself reads the top 16 bits of each key (bits
 *                 30..15) from the context, and takes a candidate's full key
 *                 from key_out, or else recomputes it from m (unchanged off
 *                 the mask), the owner's residual and its sparse buffer with
 *                 the same fp32 operations; the mask is the same either way.
 * Errors: INVALID_ARG, ALIGN, STATE (next aliases cur), HIP.
 */
int scape_step(scape_ctx* ctx, float* x, float* m, float* v, float* const* r, const uint16_t* const* g,
               const scape_mask* cur, const scape_mask* next, float* const* sparse_bufs, uint32_t* key_out,
               void* stream);

/*
 * scape_step in the interleaved layout, which groups in HBM what the step
 * reads or writes together:
 *   - the W workers' residuals and gradients as one array each, in which
 *     every 64-element word of the flat layout holds worker 0's 64 values,
 *     then worker 1's, ..., then worker W-1's.  Element j = 64*w + l
 *     (0 <= l < 64) of worker i is r_il[(w*W + i)*64 + l] and
 *     g_il[(w*W + i)*64 + l].  The dense pass then streams two worker arrays
 *     instead of 2W (measured on the 1.75B-shaped workload at W = 4: 14.3
 *     against 15.3 ms for the pass);
 *   - the parameters and the second moment as (x, v) pairs, xv[2j] = x[j] and
 *     xv[2j+1] = v[j]: the sparse update touches both at the same masked
 *     positions, and one 8-byte access per position replaces two scattered
 *     ones (measured on 17.5M positions at 1% density: 1.4-1.7 against
 *     2.1-2.5 ms).  Nothing else in the step reads x or v.
 * Same computation and results as scape_step, bit for bit.
 * Arguments as scape_step, except:
 *   xv    fp32 device array of 2*n_pad elements, updated in place (v at
 *         masked positions is written, never read);
 *   r_il  fp32 device array of n_pad*W elements, updated in place;
 *   g_il  bfloat16 bits (uint16) device array of n_pad*W elements, read only;
 * all 16-byte aligned.
 * Errors: as scape_step.
 */
int scape_step_interleaved(scape_ctx* ctx, float* xv, float* m, float* r_il, const uint16_t* g_il,
                           const scape_mask* cur, const scape_mask* next, float* const* sparse_bufs,
                           uint32_t* key_out, void* stream);

/*
 * scape_step with the W residuals in pinned host memory: CPU offloading of
 * the residual buffers with double buffering ([TS-2] Memory Optimization).
 * Same computation and results as scape_step, bit for bit.  Where the GPU
 * can address every residual array (pinned, mapped host memory; see
 * scape_set_offload_path), the dense pass reads and writes the residuals in
 * host memory itself, so PCIe carries both directions at once.  Otherwise
 * the residuals move through the GPU in chunks of 2^27 / W elements per
 * worker (512 MB of residuals per chunk, the whole n_pad if smaller): host ->
 * one of two device staging slots on that slot's copy-in stream, the dense
 * pass on `stream`, staging -> host on the slot's copy-out stream, the two
 * slots alternating so the PCIe copies of one chunk overlap the dense pass
 * and copies of the other.  The rest of the step does not touch the
 * residuals, so the last copies back overlap it.
 * The step is complete on `stream` only once every residual chunk is back.
 * Arguments as scape_step, except r_host: a host array of W pointers to
 * pinned host memory (hipHostMalloc, or a pinned torch tensor), n_pad fp32
 * each, 16-byte aligned; pageable memory also works but copies synchronously.
 * The host must not touch r_host while a step is in flight.  The first call
 * on a context allocates what only this entry point uses, kept until
 * scape_destroy: a full-key array (n_pad x 4 bytes; the selection does not
 * read candidates' residuals in host memory), and for the staged path the
 * staging slots (2 x 512 MB at most) and four copy streams (default
 * priority); that call may block like hipMalloc.
 * Errors: as scape_step, and OOM.
 */
int scape_step_offload(scape_ctx* ctx, float* x, float* m, float* v, float* const* r_host, const uint16_t* const* g,
                       const scape_mask* cur, const scape_mask* next, float* const* sparse_bufs, uint32_t* key_out,
                       void* stream);

/*
 * One dense AdamS step on W simulated workers: the baseline the pages measure
 * SCAPE's per-step speedup against ([abs]; [TS-4] Per-Step Speedup).  The
 * pages do not define it; the reading taken is plain data parallelism, in
 * which the dense all-reduce of the gradients drives the same AdamS update as
 * scape_step.  Per element j of every tensor, with mo = m[j] before the step:
 *   gbar  = ((float(g_0[j]) + float(g_1[j])) + ... + float(g_{W-1}[j])) / W
 *   m_new = beta1*mo + (1-beta1)*gbar
 *   v[j]  = beta2*mo^2 + (1-beta2)*gbar^2
 *   m[j]  = m_new
 *   x[j]  = x[j] - lr*(m_new/(sqrt(v[j]) + eps) + weight_decay*x[j])
 * No residual and no mask.  Padding elements (past the end of a tensor) are
 * not touched.  Same fp32 rules as scape_step.
 * Arguments (device, n_pad elements): x, m, v fp32 state, updated in place;
 *   g[W] bfloat16 gradient bits of each worker, read only.
 * Errors: INVALID_ARG, ALIGN, HIP.
 */
int scape_dense_step(scape_ctx* ctx, float* x, float* m, float* v, const uint16_t* const* g, void* stream);

/* scape_dense_step with the W gradients in the worker-interleaved layout of
 * scape_step_interleaved (g_il: n_pad*W bfloat16 bits, 16-byte aligned).
 * x, m and v stay separate arrays: the dense step streams every element of
 * x and v, where (x, v) pairs would only add the read of v.
 * Errors: as scape_dense_step. */
int scape_dense_step_interleaved(scape_ctx* ctx, float* x, float* m, float* v, const uint16_t* g_il, void* stream);

/*
 * Mask build alone, from first-moment statistics mtilde (fp32, n_pad): per
 * layer, the k_l positions with the largest |mtilde| (bit pattern order),
 * ties to the lower position ([TS-2] Partitioned Mask Synchronization).
 *   num_shards <= 0 or shard < 0: every layer; writes out->bits (all words),
 *     out->idx and out->block_prefix.
 *   otherwise: only the layers whose owner under num_shards shards is
 *     `shard` (the one worker's share); writes only the words of those
 *     layers in out->bits; idx and block_prefix are not touched (may be NULL)
 *     - after all shards are gathered, scape_mask_index builds them.
 * Errors: INVALID_ARG, ALIGN, HIP.
 */
int scape_mask_build(scape_ctx* ctx, const float* mtilde, int32_t num_shards, int32_t shard,
                     const scape_mask* out, void* stream);

/*
 * The "fill-in" alternative to partitioned masks, one worker at a time: the
 * per-layer top-k of |mtilde| (same rule as scape_mask_build) over every
 * layer, OR-ed into acc_bits.  [TS-2] Partitioned Mask Synchronization names
 * the union of such per-worker global masks, which fills in as workers are
 * added, as what owner-partitioned masks avoid; this entry point measures it.
 * Usage: zero acc_bits (n_pad/64 words), call once per worker with that
 * worker's first-moment candidates, then scape_mask_index on a mask whose
 * bits are acc_bits: block_prefix[n_pad/64] is the size of the union (idx
 * keeps at most k_total positions).
 * Arguments: mtilde fp32 device (n_pad); acc_bits device (n_pad/64 words),
 *   read and written.
 * Errors: INVALID_ARG, ALIGN, HIP.
 */
int scape_mask_union_add(scape_ctx* ctx, const float* mtilde, uint64_t* acc_bits, void* stream);

/* idx and block_prefix of a mask from its bits (all n_pad/64 words).  At most
 * k_total positions are stored in idx; block_prefix counts every set bit.
 * Errors: INVALID_ARG, ALIGN, HIP. */
int scape_mask_index(scape_ctx* ctx, const scape_mask* mask, void* stream);

/*
 * scape_mask_index without a context and without allocating: for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same result as scape_mask_index
 * on a mask of n_words words with at most k_cap positions stored: idx (the
 * set positions in ascending order, the first k_cap of them) and
 * block_prefix[n_words+1] (set bits before each word; the last entry counts
 * every set bit).  Its partial sums live in a static device array of the
 * library (about 64 KB, held by every GPU the library runs on until the
 * process ends), so n_words is limited to 2^25 (every layout scape_init
 * takes).  Every entry a call reads is written earlier in the same call;
 * calls that overlap on one GPU share that array and race.  It calls no
 * allocating routine.
 * Arguments: bits device (n_words words, 8-byte aligned), idx device (k_cap
 * entries, 4-byte aligned; may be NULL when k_cap = 0), block_prefix device
 * (n_words+1 entries, 4-byte aligned).
 * Errors: INVALID_ARG, ALIGN, SHAPE (n_words > 2^25), HIP.
 */
int scape_mask_index_static(const uint64_t* bits, int64_t n_words, uint32_t* idx, int64_t k_cap,
                            uint32_t* block_prefix, void* stream);

/* Pack n bytes (nonzero = set) into ceil(n/64) words, LSB first; bits past n
 * are zero.  Unpack writes n bytes of 0/1 and nothing past them.  pred needs
 * no alignment (a 16-byte aligned pred is read or written 16 bytes at a
 * time), bits 8-byte alignment.  n >= 0 (n = 0 enqueues nothing).  Errors:
 * INVALID_ARG, ALIGN, SHAPE (n >= 2^37), HIP. */
int scape_pack(const uint8_t* pred, int64_t n, uint64_t* bits, void* stream);
int scape_unpack(const uint64_t* bits, int64_t n, uint8_t* pred, void* stream);

/* out[q] = ((bufs[0][q] + bufs[1][q]) + ... + bufs[W-1][q]) / W for q < k:
 * the mean of the W sparse buffers summed in worker order, the one-GPU
 * stand-in for the all-reduce of [TS-2] Single-Buffer Second-Moment
 * Reconstruction.  bufs is a host array of W device pointers (4-byte
 * aligned); 1 <= W <= 32; k >= 0.  Errors: INVALID_ARG, ALIGN, SHAPE, HIP. */
int scape_reduce_sparse(const float* const* bufs, int32_t W, int64_t k, float* out, void* stream);

/* Measurement helper, not a step of the method: copy `bytes` from src to dst
 * (device, 16-byte aligned, not overlapping; bytes a multiple of 16) with a
 * plain one-shot kernel of the dense pass's kind (16 bytes per thread,
 * non-temporal loads and stores).  Timing it gives the stream-copy rate of
 * the GPU, the practical ceiling the step's HBM-bound kernels are compared
 * with.  bytes = 0 enqueues nothing.  Errors: INVALID_ARG, ALIGN, SHAPE, HIP. */
int scape_copy_probe(const void* src, void* dst, uint64_t bytes, void* stream);

/* Measurement helper, not a step of the method: a pass with a chosen
 * traffic shape and no other work, to compare a kernel with the rate the
 * memory system gives that shape.  It reads n_src device arrays and writes
 * n_dst device arrays (each 0..4, not both 0; host arrays of pointers and
 * widths) over n_words 64-element words: element e of array i spans
 * width[i] bytes (2, 4, 8 or 16) at byte e * width[i], so a word of it is
 * 64 * width[i] bytes.  Each lane reads its element of every source, all
 * loads issued before any is used, and writes to every destination the XOR
 * of the 32-bit parts it read (a 2-byte element zero-extended), repeated to
 * the destination's width (low half for width 2).  A destination may be a
 * source (read, then written in place).  The same one-shot, XCD-aware order
 * and non-temporal accesses as the dense pass.  n_words = 0 enqueues
 * nothing.  Errors: INVALID_ARG, ALIGN (an array not aligned to its width),
 * SHAPE, HIP. */
int scape_stream_probe(const void* const* src, const uint32_t* src_width, int32_t n_src, void* const* dst,
                       const uint32_t* dst_width, int32_t n_dst, uint64_t n_words, void* stream);

/* Optional per-phase timing of scape_step with HIP events recorded on the
 * step's stream (and on the context's update stream).  Where the dense pass
 * finishes the W-way reduction and the update itself (see
 * scape_set_update_in_dense_pass), that phase reads about 0 and the
 * selection follows the dense pass.  Otherwise the update is a pass of its
 * own: on the sampled selection path it
 * runs on the context's own stream beside the selection's record passes
 * (they share no data the other writes), starting once the key filter is
 * done, so those two phases overlap and both are measured from the end of the
 * dense pass; on the compact path (see scape_set_select_path) it follows the
 * selection on the step's stream and every phase is measured alone.
 * Phases: */
#define SCAPE_PHASE_EF_COMPACT 0    /* error feedback, candidates, compaction, statistic */
#define SCAPE_PHASE_REDUCE_UPDATE 1 /* W-way reduction, reconstruction, v/m/x update     */
#define SCAPE_PHASE_MASK_SELECT 2   /* per-layer top-k into bits                        */
#define SCAPE_PHASE_MASK_INDEX 3    /* idx and block_prefix of the new mask             */
#define SCAPE_PHASE_COUNT 4
/* enable != 0 starts recording (clearing earlier records); 0 stops. */
int scape_profile_enable(scape_ctx* ctx, int32_t enable);
/* Waits for the recorded events and returns, per phase, the summed
 * milliseconds (ms[SCAPE_PHASE_COUNT]) and the number of steps recorded. */
int scape_profile_read(scape_ctx* ctx, double* ms, int64_t* steps);

#ifdef __cplusplus
}
#endif

#endif /* SCAPE_H */
