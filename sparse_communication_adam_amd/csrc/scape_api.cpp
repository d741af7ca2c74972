// scape_api.cpp - host side of libscape: argument validation, the flat
// layout, tile tables, device workspaces, and the launch sequence of each
// entry point declared in include/scape.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "scape_internal.h"

using namespace scape;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SCAPE_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

#define SCAPE_HIP(call, what)                      \
    do {                                           \
        hipError_t e_ = (call);                    \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxFlat = int64_t(1) << 31;  // positions are uint32 and j*64 stays below 2^32

struct HostLayout {
    int32_t L = 0;
    std::vector<int64_t> n, off, k;
    int64_t n_pad = 0, k_total = 0;
};

int validate_config(const scape_config* cfg) {
    if (!cfg) return fail(SCAPE_ERR_INVALID_ARG, "config is NULL");
    if (cfg->num_layers < 1) return fail(SCAPE_ERR_SHAPE, "num_layers must be >= 1 (got %d)", cfg->num_layers);
    if (!cfg->layer_numel) return fail(SCAPE_ERR_INVALID_ARG, "layer_numel is NULL");
    if (cfg->workers < 1 || cfg->workers > SCAPE_MAX_WORKERS)
        return fail(SCAPE_ERR_INVALID_ARG, "workers must be in 1..%d (got %d)", SCAPE_MAX_WORKERS, cfg->workers);
    if (cfg->owner_shards < 0 || cfg->owner_shards > cfg->workers)
        return fail(SCAPE_ERR_INVALID_ARG, "owner_shards must be in 0..workers (got %d)", cfg->owner_shards);
    if (cfg->keep_den < 1 || cfg->keep_num > cfg->keep_den)
        return fail(SCAPE_ERR_INVALID_ARG, "keep must satisfy 0 <= keep_num <= keep_den, keep_den >= 1 (got %u/%u)",
                    cfg->keep_num, cfg->keep_den);
    if (!(cfg->beta1 >= 0.0f && cfg->beta1 < 1.0f) || !(cfg->beta2 >= 0.0f && cfg->beta2 < 1.0f))
        return fail(SCAPE_ERR_INVALID_ARG, "beta1 and beta2 must be in [0, 1)");
    if (!(cfg->lr == cfg->lr) || !(cfg->eps == cfg->eps) || !(cfg->weight_decay == cfg->weight_decay))
        return fail(SCAPE_ERR_INVALID_ARG, "lr, eps and weight_decay must not be NaN");
    int64_t cur = 0;
    for (int32_t l = 0; l < cfg->num_layers; ++l) {
        const int64_t n = cfg->layer_numel[l];
        if (n < 0) return fail(SCAPE_ERR_SHAPE, "layer %d has negative size %lld", l, (long long)n);
        if (n >= kMaxFlat) return fail(SCAPE_ERR_SHAPE, "layer %d is too large (%lld)", l, (long long)n);
        cur += (n + 63) / 64 * 64;
        if (cur >= kMaxFlat)
            return fail(SCAPE_ERR_SHAPE, "padded total exceeds 2^31 - 1 elements at layer %d", l);
    }
    return SCAPE_OK;
}

int64_t kept_count(int64_t n, uint32_t num, uint32_t den) {
    // n < 2^31 and num < 2^32: the product fits in 64 bits
    return (int64_t)(((uint64_t)n * num + den - 1) / den);
}

void build_layout(const scape_config* cfg, HostLayout* h) {
    h->L = cfg->num_layers;
    h->n.assign(cfg->layer_numel, cfg->layer_numel + h->L);
    h->off.resize(h->L);
    h->k.resize(h->L);
    int64_t cur = 0, kt = 0;
    for (int32_t l = 0; l < h->L; ++l) {
        h->off[l] = cur;
        cur += (h->n[l] + 63) / 64 * 64;
        h->k[l] = kept_count(h->n[l], cfg->keep_num, cfg->keep_den);
        if (h->k[l] > h->n[l]) h->k[l] = h->n[l];
        kt += h->k[l];
    }
    h->n_pad = cur;
    h->k_total = kt;
}

// Shard of an even split of [0, n_pad) into P parts holding the layer
// midpoint off + n/2, i.e. floor(P * (2*off + n) / (2*n_pad)), capped.
void owner_map(const HostLayout& h, int32_t P, int32_t* owner) {
    for (int32_t l = 0; l < h.L; ++l) {
        if (h.n_pad == 0) {
            owner[l] = 0;
            continue;
        }
        const uint64_t num = (uint64_t)P * (uint64_t)(2 * h.off[l] + h.n[l]);
        int64_t s = (int64_t)(num / (uint64_t)(2 * h.n_pad));
        owner[l] = (int32_t)(s > P - 1 ? P - 1 : s);
    }
}

struct ProfSlot {
    hipEvent_t ev[SCAPE_PHASE_COUNT + 1];
    bool pending;
    bool serial;  // the update ran after the selection on the step's stream
};

constexpr int kProfSlots = 64;

}  // namespace

// Residual offload: two staging slots, each with its own copy streams, of
// 512 MB each (W residual chunks).  Larger copies move faster over PCIe: on
// the 1.75B workload (W = 4) chunks of 2^16, 2^18, 2^19 and 2^21 words took
// about 1.5, 1.25, 0.97 and 0.94 s per step.  More slots (3 or 4) were not
// faster.
// With the update in the dense pass switched on, the dense pass touches x,
// v and m at the masked elements only where the mask keeps at most
// 1 / kFuseMaxDensityInv of the elements, and streams them whole on denser
// masks (SCAPE_FUSE_DENSE 0: denser masks keep the separate update).
#ifndef SCAPE_FUSE_MAX_DENSITY_INV
#define SCAPE_FUSE_MAX_DENSITY_INV 32
#endif
#ifndef SCAPE_FUSE_DENSE
#define SCAPE_FUSE_DENSE 1
#endif
constexpr uint64_t kFuseMaxDensityInv = SCAPE_FUSE_MAX_DENSITY_INV;
constexpr int kOffloadSlots = 2;
constexpr size_t kOffloadSlotBytes = size_t(512) << 20;
constexpr uint32_t kOffloadMinChunkWords = 1u << 12;

struct scape_ctx {
    int device = 0;
    scape_config cfg{};
    HostLayout lay;
    int32_t P = 1;
    std::vector<int32_t> owner;
    std::vector<TileDesc> tiles;
    std::vector<uint32_t> layer_tile0;  // first tile of each layer (L+1 entries)
    std::vector<SegDesc> segs;
    std::vector<uint32_t> layer_seg0;   // first record segment of each layer (L+1 entries)
    uint32_t n_words = 0;
    uint32_t n_index_blocks = 0;
    uint32_t cand_cap = 0;
    // device workspaces
    LayerDesc* d_layers = nullptr;
    TileDesc* d_tiles = nullptr;
    uint32_t* d_hist = nullptr;
    SelState* d_sel = nullptr;
    SegDesc* d_segs = nullptr;
    uint32_t* d_layer_seg0 = nullptr;
    uint32_t* d_seg_fill = nullptr;   // per segment: records
    uint32_t* d_seg_above = nullptr;  // per segment: keys above the window
    uint64_t* d_union_bits = nullptr;  // one worker's mask before it is OR-ed into a fill-in union
    VblockDesc* d_vb = nullptr;       // record blocks
    uint32_t* d_vb_count = nullptr;   // records per block
    size_t vb_cap = 0;
    uint32_t* d_totals = nullptr;
    uint32_t* d_miss = nullptr;  // set when a layer's threshold fell outside its sampled window
    uint64_t* d_cand = nullptr;
    uint16_t* d_key16 = nullptr;      // statistic keys, bits 30..15 (what the selection reads)
    uint32_t* d_key32 = nullptr;      // full statistic keys, for the offloaded step
    uint32_t* d_block_sums = nullptr;
    uint16_t* d_word_info = nullptr;  // per word: owner << 8 | elements inside the layer
    uint32_t* d_counts = nullptr;     // per layer: sampled keys
    uint32_t* d_ovf = nullptr;        // per layer: records lost to the record space in the key filter
    float* d_m_stash = nullptr;       // m at the current mask's positions, compacted (k_total)
    // the compact selection path: per layer its whole record space, and
    // [ticket | record count | bit count] rows of L counters
    SegDesc* d_lspace = nullptr;
    uint32_t* d_lcount = nullptr;
    unsigned long long* d_ltick = nullptr;  // the filter's per-layer tickets
    float* d_dummy = nullptr;               // 16 bytes no kernel writes (a safe load address)
    int32_t select_path = SCAPE_SELECT_PATH_AUTO;
    bool update_in_dense = true;            // scape_set_update_in_dense_pass
    int32_t offload_path = SCAPE_OFFLOAD_PATH_AUTO;  // scape_set_offload_path
    // the update runs on its own stream beside the mask selection
    hipStream_t s_upd = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    // residual offload (made by the first offloaded step): staging slots of W
    // chunks, each slot with its own copy-in and copy-out stream
    float* d_stage = nullptr;         // [kOffloadSlots][W][chunk_words * 64]
    uint32_t chunk_words = 0;
    hipStream_t s_in[kOffloadSlots] = {}, s_out[kOffloadSlots] = {};
    hipEvent_t ev_in[kOffloadSlots] = {}, ev_k[kOffloadSlots] = {}, ev_out[kOffloadSlots] = {};
    bool offload_ready = false;
    // profiling
    bool prof_on = false;
    ProfSlot prof[kProfSlots]{};
    bool prof_events = false;
    int prof_next = 0;
    double prof_ms[SCAPE_PHASE_COUNT] = {0, 0, 0, 0};
    int64_t prof_steps = 0;
    size_t ws_bytes = 0;  // device memory the context holds
};

namespace {

void free_ctx(scape_ctx* c) {
    hipFree(c->d_layers);
    hipFree(c->d_tiles);
    hipFree(c->d_hist);
    hipFree(c->d_sel);
    hipFree(c->d_segs);
    hipFree(c->d_lspace);
    hipFree(c->d_lcount);
    hipFree(c->d_ltick);
    hipFree(c->d_dummy);
    hipFree(c->d_layer_seg0);
    hipFree(c->d_seg_fill);
    hipFree(c->d_seg_above);
    hipFree(c->d_union_bits);
    hipFree(c->d_vb);
    hipFree(c->d_vb_count);
    hipFree(c->d_totals);
    hipFree(c->d_miss);
    hipFree(c->d_cand);
    hipFree(c->d_key16);
    hipFree(c->d_key32);
    hipFree(c->d_block_sums);
    hipFree(c->d_word_info);
    hipFree(c->d_counts);
    hipFree(c->d_ovf);
    hipFree(c->d_m_stash);
    hipFree(c->d_stage);
    for (int b = 0; b < kOffloadSlots; ++b) {
        if (c->ev_in[b]) hipEventDestroy(c->ev_in[b]);
        if (c->ev_k[b]) hipEventDestroy(c->ev_k[b]);
        if (c->ev_out[b]) hipEventDestroy(c->ev_out[b]);
        if (c->s_in[b]) hipStreamDestroy(c->s_in[b]);
        if (c->s_out[b]) hipStreamDestroy(c->s_out[b]);
    }
    if (c->ev_fork) hipEventDestroy(c->ev_fork);
    if (c->ev_join) hipEventDestroy(c->ev_join);
    if (c->s_upd) hipStreamDestroy(c->s_upd);
    if (c->prof_events)
        for (auto& s : c->prof)
            for (auto& e : s.ev) hipEventDestroy(e);
    delete c;
}

template <typename T>
int dev_alloc(scape_ctx* c, T** p, size_t count, const char* what) {
    const size_t bytes = count * sizeof(T) > 0 ? count * sizeof(T) : 16;
    hipError_t e = hipMalloc((void**)p, bytes);
    if (e == hipErrorOutOfMemory) return fail(SCAPE_ERR_OOM, "out of device memory allocating %s (%zu bytes)", what, bytes);
    if (e != hipSuccess) return hip_fail(e, what);
    c->ws_bytes += bytes;
    return SCAPE_OK;
}

int check_device(const scape_ctx* ctx) {
    int dev = -1;
    SCAPE_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev != ctx->device)
        return fail(SCAPE_ERR_STATE, "context was created on device %d but device %d is current", ctx->device, dev);
    return SCAPE_OK;
}

int check_mask(const scape_mask* m, bool need_index, const char* name) {
    if (!m) return fail(SCAPE_ERR_INVALID_ARG, "%s is NULL", name);
    if (!m->bits) return fail(SCAPE_ERR_INVALID_ARG, "%s->bits is NULL", name);
    if (!aligned(m->bits, 8)) return fail(SCAPE_ERR_ALIGN, "%s->bits must be 8-byte aligned", name);
    if (need_index) {
        if (!m->idx || !m->block_prefix) return fail(SCAPE_ERR_INVALID_ARG, "%s->idx/block_prefix is NULL", name);
        if (!aligned(m->idx, 4) || !aligned(m->block_prefix, 4))
            return fail(SCAPE_ERR_ALIGN, "%s->idx/block_prefix must be 4-byte aligned", name);
    }
    return SCAPE_OK;
}

// Record the event that closes `phase` (0..COUNT-1) or opens the step (-1).
void prof_mark(scape_ctx* c, int slot, int point, hipStream_t s) {
    if (slot >= 0) hipEventRecord(c->prof[slot].ev[point], s);
}

void prof_collect(scape_ctx* c, int slot) {
    ProfSlot& p = c->prof[slot];
    if (!p.pending) return;
    hipEventSynchronize(p.ev[SCAPE_PHASE_COUNT]);
    // points: 0 start, 1 end of the dense pass (where the update and the
    // selection fork), 2 end of the update, 3 end of the selection, 4 end of
    // the index and the join.  The update and the selection run side by side,
    // so both are measured from point 1; in a serial step the update follows
    // the selection (3 -> 2) and the index follows the update (2 -> 4).
    static const int from[SCAPE_PHASE_COUNT] = {0, 1, 1, 3};
    static const int from_serial[SCAPE_PHASE_COUNT] = {0, 3, 1, 2};
    static const int to[SCAPE_PHASE_COUNT] = {1, 2, 3, 4};
    for (int i = 0; i < SCAPE_PHASE_COUNT; ++i) {
        float ms = 0.0f;
        const int a = p.serial ? from_serial[i] : from[i];
        if (hipEventElapsedTime(&ms, p.ev[a], p.ev[to[i]]) == hipSuccess) c->prof_ms[i] += ms;
    }
    c->prof_steps += 1;
    p.pending = false;
}

int prof_begin(scape_ctx* c) {
    if (!c->prof_on) return -1;
    const int slot = c->prof_next;
    c->prof_next = (c->prof_next + 1) % kProfSlots;
    prof_collect(c, slot);  // the ring wrapped: fold the old record first
    c->prof[slot].pending = true;
    c->prof[slot].serial = false;
    return slot;
}

// Mask selection over layers [la, la+nl) and tiles [ta, tb), from 16-bit keys
// and the source of candidates' full keys, bits into `bits`.
// `fork`, when given, is recorded on `s` once the key filter is queued (at
// once if there is nothing to select): the step's update starts there.
// Whether the layers [la, la + nl) take the compact path: each of them at
// most kCompactMaxLayer elements, unless the caller chose a path.
bool compact_range(const scape_ctx* c, int32_t la, int32_t nl) {
    if (c->select_path != SCAPE_SELECT_PATH_AUTO) return c->select_path == SCAPE_SELECT_PATH_COMPACT;
    for (int32_t l = la; l < la + nl; ++l)
        if (c->lay.n[l] > kCompactMaxLayer) return false;
    return true;
}

// The compact path: two launches.  The update only waits for the dense pass,
// so its fork is recorded first.
int run_select_compact(scape_ctx* c, int32_t la, int32_t nl, uint32_t ta, uint32_t tb, const uint16_t* key,
                       const KeySource& ks, uint64_t* bits, hipStream_t s, hipEvent_t fork) {
    (void)la;
    (void)nl;
    if (fork) SCAPE_HIP(hipEventRecord(fork, s), "fork");
    const uint32_t nt = tb - ta;
    if (nt == 0) return SCAPE_OK;  // only empty layers: no bits to set
    const TileDesc* tiles = c->d_tiles + ta;
    const uint32_t L = (uint32_t)c->lay.L;
    uint32_t* ticket = c->d_lcount;
    uint32_t* lrec = c->d_lcount + L;
    uint32_t* labove = c->d_lcount + 2 * (size_t)L;
    // split the tiles until the launches have about kCompactBlocks workgroups
    auto parts_for = [&](uint32_t target, uint32_t most) {
        return std::max<uint32_t>(1u, std::min<uint32_t>(most, (target + nt - 1) / nt));
    };
    SCAPE_HIP(launch_compact_hist(s, tiles, nt, parts_for(kCompactHistBlocks, kCompactHistParts), c->d_layers, key,
                                  c->d_hist, c->d_sel, ticket, lrec, labove, c->d_miss),
              "compact_hist");
    SCAPE_HIP(launch_compact_filter(s, tiles, nt, parts_for(kCompactFilterBlocks, kCompactFilterParts), c->d_layers,
                                    c->d_lspace, c->d_sel, key, ks, bits, c->d_cand, c->d_ltick, lrec, labove,
                                    c->d_miss),
              "compact_filter");
    return SCAPE_OK;
}

// `zero`: ranges the caller needs zeroed before the selection (the mask
// build's histogram rows); the sampled path zeroes them with its own counters
// in one launch.
int run_select(scape_ctx* c, int32_t la, int32_t nl, uint32_t ta, uint32_t tb, const uint16_t* key,
               const KeySource& ks, uint64_t* bits, hipStream_t s, hipEvent_t fork = nullptr,
               ZeroRanges zero = ZeroRanges{}) {
    if (compact_range(c, la, nl)) {
        SCAPE_HIP(launch_zero_ranges(s, zero), "zero");
        return run_select_compact(c, la, nl, ta, tb, key, ks, bits, s, fork);
    }
    const TileDesc* tiles = c->d_tiles + ta;
    const uint32_t nt = tb - ta;
    const uint32_t sa = c->layer_seg0[la], ns = c->layer_seg0[la + nl] - sa;
    if (ns == 0) {  // every layer in the range is empty: no bits to set
        SCAPE_HIP(launch_zero_ranges(s, zero), "zero");
        if (fork) SCAPE_HIP(hipEventRecord(fork, s), "fork");
        return SCAPE_OK;
    }
    uint32_t* sample_count = c->d_counts;
    if (zero.count > kZeroRangesMax - 4) return fail(SCAPE_ERR_STATE, "too many ranges to zero");
    zero.add(c->d_seg_fill + sa, (uint64_t)ns);
    zero.add(c->d_seg_above + sa, (uint64_t)ns);
    zero.add(sample_count + la, (uint64_t)nl);
    zero.add(c->d_ovf + la, (uint64_t)nl);
    SCAPE_HIP(launch_zero_ranges(s, zero), "zero");
    SCAPE_HIP(launch_sample_hist(s, tiles, nt, c->d_layers, key, c->d_hist, sample_count), "sample_hist");
    SCAPE_HIP(launch_estimate(s, la, nl, c->d_layers, c->d_hist, sample_count, c->d_sel, c->d_miss), "estimate");
    SCAPE_HIP(launch_filter(s, tiles, nt, c->d_layers, c->d_segs, c->d_sel, key, bits, c->d_seg_fill, c->d_cand,
                            c->d_seg_above, c->d_hist),
              "filter");
    if (fork) SCAPE_HIP(hipEventRecord(fork, s), "fork");
    // the filter counted the records' first digits; overflowed record spaces
    // are flagged here, and the threshold bucket of each layer found next
    SCAPE_HIP(launch_cand_scan(s, sa, ns, c->d_segs, c->d_seg_fill, c->d_vb, c->d_vb_count, c->d_totals, false,
                               c->d_ovf, c->d_sel, c->d_miss),
              "cand_scan");
    SCAPE_HIP(launch_select_first(s, la, nl, true, c->d_layers, c->d_layer_seg0, c->d_hist, c->d_sel,
                                  c->d_seg_above, c->d_seg_fill, c->d_ovf, c->d_miss),
              "select_first");
    // sampling misses and lost records: full histogram, exact bucket,
    // reclassification
    SCAPE_HIP(launch_hist_full(s, tiles, nt, c->d_layers, c->d_sel, key, c->d_hist, c->d_miss), "hist_full");
    SCAPE_HIP(launch_select_first(s, la, nl, false, c->d_layers, c->d_layer_seg0, c->d_hist, c->d_sel,
                                  c->d_seg_above, c->d_seg_fill, c->d_ovf, c->d_miss),
              "select_first");
    SCAPE_HIP(launch_filter_exact(s, tiles, nt, c->d_layers, c->d_segs, c->d_sel, key, bits, c->d_seg_fill,
                                  c->d_cand, c->d_seg_above, c->d_miss),
              "filter_exact");
    // radix passes with shrinking record sets, then the final marking; a layer
    // whose exact bucket still did not fit its record space is decided by
    // passes over its keys instead
    SCAPE_HIP(launch_cand_scan(s, sa, ns, c->d_segs, c->d_seg_fill, c->d_vb, c->d_vb_count, c->d_totals, true,
                               c->d_ovf, c->d_sel, c->d_miss),
              "cand_scan");
    for (uint32_t phase = kPhaseKey2; phase <= kPhasePos3; ++phase) {
        SCAPE_HIP(launch_cand_pass(s, phase, c->d_vb, c->d_vb_count, c->d_totals, c->d_layers, c->d_sel, ks, c->d_cand,
                                   c->d_hist, bits, tiles, nt, key, c->d_miss),
                  "cand_pass");
        SCAPE_HIP(launch_select_next(s, phase, la, nl, c->d_hist, c->d_sel), "select_next");
    }
    SCAPE_HIP(launch_cand_pass(s, kPhaseDone, c->d_vb, c->d_vb_count, c->d_totals, c->d_layers, c->d_sel, ks, c->d_cand,
                               c->d_hist, bits, tiles, nt, key, c->d_miss),
              "cand_pass");
    return SCAPE_OK;
}

int run_index(scape_ctx* c, const scape_mask* mk, hipStream_t s) {
    if (c->n_words > 0 && c->n_words <= kIndexSmallMaxWords) {
        SCAPE_HIP(launch_index_small(s, mk->bits, c->n_words, c->d_block_sums, mk->idx, (uint32_t)c->lay.k_total,
                                     mk->block_prefix),
                  "index_small");
        return SCAPE_OK;
    }
    SCAPE_HIP(launch_index_count(s, mk->bits, c->n_words, c->d_block_sums), "index_count");
    SCAPE_HIP(launch_index_scan(s, c->d_block_sums, c->n_index_blocks), "index_scan");
    SCAPE_HIP(launch_index_emit(s, mk->bits, c->n_words, c->d_block_sums, mk->idx, (uint32_t)c->lay.k_total,
                                mk->block_prefix),
              "index_emit");
    return SCAPE_OK;
}

// The dense pass with the residuals in pinned host memory (Memory
// Optimization, gist.science Technical Summary s.2: CPU offloading with double
// buffering).  Words are independent in the dense pass, so it runs chunk by
// chunk on the step's stream with every pointer offset to the chunk; the W
// residual chunks move host -> staging slot on the slot's copy-in stream and
// back on its copy-out stream, the slots taken in turn so that the copies of
// one chunk overlap the dense pass of another.  The events order, per slot:
// copy in -> dense pass -> copy out -> the next copy into that slot.
int ef_offload(scape_ctx* c, const WorkerPtrs& wp, float* const* r_host, const StepScalars& sc, const float* m,
               const scape_mask* cur, uint32_t k_cap, uint16_t* key16, uint32_t* key32, hipStream_t s) {
    const int W = c->cfg.workers;
    const uint32_t cw = c->chunk_words;
    const size_t slot_elems = (size_t)cw * 64;
    uint32_t chunk = 0;
    for (uint32_t w0 = 0; w0 < c->n_words; w0 += cw, ++chunk) {
        const uint32_t nw = std::min(cw, c->n_words - w0);
        const int b = (int)(chunk % kOffloadSlots);
        const size_t j0 = (size_t)w0 * 64, bytes = (size_t)nw * 64 * sizeof(float);
        float* stage = c->d_stage + (size_t)b * W * slot_elems;
        SCAPE_HIP(hipStreamWaitEvent(c->s_in[b], c->ev_out[b], 0), "offload wait");
        for (int i = 0; i < W; ++i)
            SCAPE_HIP(hipMemcpyAsync(stage + (size_t)i * slot_elems, r_host[i] + j0, bytes, hipMemcpyHostToDevice,
                                     c->s_in[b]),
                      "offload copy in");
        SCAPE_HIP(hipEventRecord(c->ev_in[b], c->s_in[b]), "offload event");
        SCAPE_HIP(hipStreamWaitEvent(s, c->ev_in[b], 0), "offload wait");
        WorkerPtrs cp = wp;  // one array per worker (word stride 64)
        for (int i = 0; i < W; ++i) {
            cp.r[i] = stage + (size_t)i * slot_elems;
            cp.g[i] = wp.g[i] + j0;
        }
        // the first chunk's pass also zeroes the histogram rows
        SCAPE_HIP(launch_ef_compact(s, c->d_word_info + w0, nw, cp, sc, const_cast<float*>(m) + j0, cur->bits + w0,
                                    cur->block_prefix + w0, k_cap, key16 + j0, key32 + j0, c->d_m_stash,
                                    chunk == 0 ? c->d_hist : nullptr,
                                    chunk == 0 ? (uint32_t)c->lay.L * kHistBins : 0u, 0, nullptr, nullptr,
                                    c->d_dummy),
                  "ef_compact");
        SCAPE_HIP(hipEventRecord(c->ev_k[b], s), "offload event");
        SCAPE_HIP(hipStreamWaitEvent(c->s_out[b], c->ev_k[b], 0), "offload wait");
        for (int i = 0; i < W; ++i)
            SCAPE_HIP(hipMemcpyAsync(r_host[i] + j0, stage + (size_t)i * slot_elems, bytes, hipMemcpyDeviceToHost,
                                     c->s_out[b]),
                      "offload copy out");
        SCAPE_HIP(hipEventRecord(c->ev_out[b], c->s_out[b]), "offload event");
    }
    return SCAPE_OK;
}

// The offloaded step's resources, made by its first call on a context: the
// full-key array (without the residuals on the device, the selection cannot
// recompute candidates' keys), the staging slots, and each slot's copy
// streams and events (default priority; the events only order work).
// Whatever a failed attempt made is kept and freed with the context.
// What the offloaded step needs: the full-key array always, the staging
// slots and copy streams only for the staged path.
int ensure_offload(scape_ctx* c, bool staging) {
    if (c->n_words == 0) return SCAPE_OK;
    int rc;
    if (!c->d_key32 && (rc = dev_alloc(c, &c->d_key32, (size_t)c->lay.n_pad, "full statistic keys"))) return rc;
    if (c->offload_ready || !staging) return SCAPE_OK;
    c->chunk_words = std::min<uint32_t>(
        c->n_words, std::max<uint32_t>(kOffloadMinChunkWords, (uint32_t)(kOffloadSlotBytes / ((size_t)c->cfg.workers *
                                                                                             64 * sizeof(float)))));
    if (!c->d_stage && (rc = dev_alloc(c, &c->d_stage, (size_t)kOffloadSlots * c->cfg.workers * c->chunk_words * 64,
                                       "offload staging")))
        return rc;
    hipError_t e = hipSuccess;
    for (int b = 0; b < kOffloadSlots && e == hipSuccess; ++b) {
        if (!c->s_in[b]) e = hipStreamCreateWithFlags(&c->s_in[b], hipStreamNonBlocking);
        if (e == hipSuccess && !c->s_out[b]) e = hipStreamCreateWithFlags(&c->s_out[b], hipStreamNonBlocking);
        if (e == hipSuccess && !c->ev_in[b]) e = hipEventCreateWithFlags(&c->ev_in[b], hipEventDisableTiming);
        if (e == hipSuccess && !c->ev_k[b]) e = hipEventCreateWithFlags(&c->ev_k[b], hipEventDisableTiming);
        if (e == hipSuccess && !c->ev_out[b]) {
            e = hipEventCreateWithFlags(&c->ev_out[b], hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventRecord(c->ev_out[b], c->s_out[b]);  // every slot starts free
        }
    }
    if (e != hipSuccess) return hip_fail(e, "creating offload streams and events");
    c->offload_ready = true;
    return SCAPE_OK;
}

// The address the GPU reaches host memory at p by, if p lies in pinned host
// memory mapped for the device (with unified addressing, p itself).  A
// failed query leaves no error behind for the next launch check.
bool host_device_pointer(float* p, float** dev) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess || d == nullptr) {
        (void)hipGetLastError();
        return false;
    }
    *dev = static_cast<float*>(d);
    return true;
}

// Where the W residuals and gradients are: one device array per worker, one
// pinned host array per worker (residuals; the offloaded step), or one device
// array each holding the W workers' 64 values of every word in turn (the
// interleaved layout: r[0] and g[0] are its base pointers; x then holds the
// (x, v) pairs and v is not used).
enum class WorkerLayout { kSeparate, kHostResiduals, kInterleaved };

int step_common(scape_ctx* ctx, float* x, float* m, float* v, float* const* r, const uint16_t* const* g,
                const scape_mask* cur, const scape_mask* next, float* const* sparse_bufs, uint32_t* key_out,
                void* stream, WorkerLayout wl) {
    const bool r_on_host = wl == WorkerLayout::kHostResiduals;
    const bool il = wl == WorkerLayout::kInterleaved;
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    if (il) {  // x holds the (x, v) pairs; there is no separate v
        if (!x || !m) return fail(SCAPE_ERR_INVALID_ARG, "xv and m must not be NULL");
        if (!aligned(x, 16) || !aligned(m, 16)) return fail(SCAPE_ERR_ALIGN, "xv and m must be 16-byte aligned");
    } else {
        if (!x || !m || !v) return fail(SCAPE_ERR_INVALID_ARG, "x, m and v must not be NULL");
        if (!aligned(x, 16) || !aligned(m, 16) || !aligned(v, 16))
            return fail(SCAPE_ERR_ALIGN, "x, m and v must be 16-byte aligned");
    }
    if (!r || !g || !sparse_bufs) return fail(SCAPE_ERR_INVALID_ARG, "r, g and sparse_bufs must not be NULL");
    const int W = ctx->cfg.workers;
    for (int i = 0; i < W; ++i) {
        if (!il || i == 0) {
            if (!r[i] || !g[i]) return fail(SCAPE_ERR_INVALID_ARG, "r[%d] or g[%d] is NULL", i, i);
            if (!aligned(r[i], 16) || !aligned(g[i], 16))
                return fail(SCAPE_ERR_ALIGN, "r[%d] and g[%d] must be 16-byte aligned", i, i);
        }
        if (ctx->lay.k_total > 0) {
            if (!sparse_bufs[i]) return fail(SCAPE_ERR_INVALID_ARG, "sparse_bufs[%d] is NULL", i);
            if (!aligned(sparse_bufs[i], 4)) return fail(SCAPE_ERR_ALIGN, "sparse_bufs[%d] must be 4-byte aligned", i);
        }
    }
    if (key_out && !aligned(key_out, 16)) return fail(SCAPE_ERR_ALIGN, "key_out must be 16-byte aligned");
    int rc;
    if ((rc = check_mask(cur, true, "cur")) || (rc = check_mask(next, true, "next"))) return rc;
    if (cur->bits == next->bits || cur->idx == next->idx || cur->block_prefix == next->block_prefix)
        return fail(SCAPE_ERR_STATE, "next must not alias cur (the mask built now is used at the next step)");
    if ((rc = check_device(ctx))) return rc;
    // Residuals in host memory the GPU can address (pinned by hipHostMalloc
    // or a pinned torch tensor) are read and written by the dense pass itself
    // over PCIe, reads and writes in flight together; otherwise they move
    // through the staging slots.
    float* r_dev[SCAPE_MAX_WORKERS] = {};
    bool direct = false;
    if (r_on_host && ctx->offload_path == SCAPE_OFFLOAD_PATH_AUTO && ctx->n_words > 0) {
        direct = true;
        for (int i = 0; i < W && direct; ++i) direct = host_device_pointer(r[i], &r_dev[i]);
    }
    if (r_on_host && (rc = ensure_offload(ctx, !direct))) return rc;

    hipStream_t s = (hipStream_t)stream;
    WorkerPtrs wp{};
    wp.ws = il ? 64u * (uint32_t)W : 64u;
    for (int i = 0; i < W; ++i) {
        wp.r[i] = r_on_host ? r_dev[i] : il ? r[0] + 64 * i : r[i];
        wp.g[i] = il ? g[0] + 64 * i : g[i];
        wp.b[i] = ctx->lay.k_total > 0 ? sparse_bufs[i] : nullptr;
    }
    StepScalars sc;
    sc.beta1 = ctx->cfg.beta1;
    sc.beta2 = ctx->cfg.beta2;
    sc.c1 = 1.0f - ctx->cfg.beta1;
    sc.c2 = 1.0f - ctx->cfg.beta2;
    sc.lr = ctx->cfg.lr;
    sc.eps = ctx->cfg.eps;
    sc.wd = ctx->cfg.weight_decay;
    sc.W = W;
    // The selection reads 16-bit keys.  Candidates' full keys come from
    // key_out when the caller asks for the keys, from the context's full-key
    // array when the residuals are on the host, and otherwise are recomputed
    // from m, the owner's residual and its sparse buffer.
    uint32_t* key32 = key_out ? key_out : (r_on_host ? ctx->d_key32 : nullptr);
    KeySource ks{};
    ks.key32 = key32;
    ks.m = m;
    ks.ws = wp.ws;
    for (int i = 0; i < W; ++i) {
        ks.r[i] = wp.r[i];
        ks.b[i] = wp.b[i];
    }
    ks.cur_bits = cur->bits;
    ks.cur_prefix = cur->block_prefix;
    ks.k_cap = (uint32_t)ctx->lay.k_total;
    ks.beta1 = sc.beta1;
    ks.c1 = sc.c1;
    const uint32_t k_cap = (uint32_t)ctx->lay.k_total;
    const uint32_t n_tiles = (uint32_t)ctx->tiles.size();
    const int32_t L = ctx->lay.L;

    const int slot = prof_begin(ctx);
    prof_mark(ctx, slot, 0, s);  // the first phase brackets the dense pass alone
    // The dense pass also zeroes the selection's histogram rows.  Where the
    // context asks for it and the residuals are on the device, it also
    // finishes the update at the current mask's positions: it holds every
    // worker's candidate of an element, so the W-way mean needs no second
    // pass over the sparse buffers, and the update's x / v / m accesses ride
    // on the streaming pass instead of competing with the selection.  On a
    // sparse mask only the masked elements' x, v and m are touched; on a
    // denser one (several positions per 64-element word) scattered accesses
    // to them cost the pass more than the separate update takes (measured
    // at a kept fraction of 1/10), so there the pass streams x, v and m
    // whole and writes back the unmasked elements' old values.
    const bool sparse_mask = (uint64_t)k_cap * kFuseMaxDensityInv <= (uint64_t)ctx->lay.n_pad;
    const bool fuse = ctx->update_in_dense && !r_on_host && (sparse_mask || SCAPE_FUSE_DENSE);
    const int upd = !fuse ? 0 : sparse_mask ? (il ? 2 : 1) : (il ? 4 : 3);
    if (r_on_host && !direct) {
        if ((rc = ef_offload(ctx, wp, r, sc, m, cur, k_cap, ctx->d_key16, key32, s))) return rc;
    } else {
        SCAPE_HIP(launch_ef_compact(s, ctx->d_word_info, ctx->n_words, wp, sc, m, cur->bits, cur->block_prefix,
                                    k_cap, ctx->d_key16, key32, ctx->d_m_stash, ctx->d_hist,
                                    (uint32_t)L * kHistBins, upd, x, v, ctx->d_dummy),
                  "ef_compact");
    }
    prof_mark(ctx, slot, 1, s);
    if (fuse) {
        // The update changed x, v and m on the current mask only; the
        // selection reads m off it, and follows on `stream`.
        if (slot >= 0) ctx->prof[slot].serial = true;
        if ((rc = run_select(ctx, 0, L, 0, n_tiles, ctx->d_key16, ks, next->bits, s))) return rc;
        prof_mark(ctx, slot, 3, s);
        prof_mark(ctx, slot, 2, s);  // (the update ran inside the dense pass)
        if ((rc = run_index(ctx, next, s))) return rc;
        prof_mark(ctx, slot, 4, s);
        return SCAPE_OK;
    }
    if (compact_range(ctx, 0, L) && !r_on_host) {
        // The compact selection is two short launches: forking the update
        // onto its own stream costs more in events than it overlaps, so the
        // update follows the selection on `stream`.
        if (slot >= 0) ctx->prof[slot].serial = true;
        if ((rc = run_select(ctx, 0, L, 0, n_tiles, ctx->d_key16, ks, next->bits, s))) return rc;
        prof_mark(ctx, slot, 3, s);
        SCAPE_HIP(launch_reduce_update(s, wp, sc, x, m, v, il, cur->idx, cur->block_prefix, ctx->d_m_stash,
                                       ctx->n_words, (uint32_t)ctx->lay.n_pad, k_cap),
                  "reduce_update");
        prof_mark(ctx, slot, 2, s);
        if ((rc = run_index(ctx, next, s))) return rc;
        prof_mark(ctx, slot, 4, s);
        return SCAPE_OK;
    }
    // The update touches x, v, and m on the mask only; the selection reads
    // the keys, m off the mask, the owner's residual and the sparse buffers.
    // Nothing one writes is read by the other, so the update runs on its own
    // stream beside the selection, and `stream` waits for it at the end.  It
    // starts after the key filter: the sampling and filter passes stream the
    // keys and run best alone.  The latency-bound record passes that follow
    // are slowed by the update's scattered traffic, but forking the update
    // only after the whole selection measured slower where the dense pass
    // lands at its slow placement (and no faster elsewhere).
    rc = run_select(ctx, 0, L, 0, n_tiles, ctx->d_key16, ks, next->bits, s, ctx->ev_fork);
    if (rc) return rc;  // nothing was queued on the update's stream
    SCAPE_HIP(hipStreamWaitEvent(ctx->s_upd, ctx->ev_fork, 0), "fork");
    SCAPE_HIP(launch_reduce_update(ctx->s_upd, wp, sc, x, m, v, il, cur->idx, cur->block_prefix, ctx->d_m_stash,
                                   ctx->n_words, (uint32_t)ctx->lay.n_pad, k_cap),
              "reduce_update");
    prof_mark(ctx, slot, 2, ctx->s_upd);
    const hipError_t je = hipEventRecord(ctx->ev_join, ctx->s_upd);
    if (je != hipSuccess) {  // no event to join on: the update must still not outlive the step
        hipStreamSynchronize(ctx->s_upd);
        return hip_fail(je, "join");
    }
    prof_mark(ctx, slot, 3, s);
    rc = run_index(ctx, next, s);
    // join even after a failed launch
    SCAPE_HIP(hipStreamWaitEvent(s, ctx->ev_join, 0), "join");
    if (rc) return rc;
    if (r_on_host && !direct && ctx->n_words > 0) {
        // the step completes on `stream` only once every residual chunk is home
        for (int b = 0; b < kOffloadSlots; ++b) SCAPE_HIP(hipStreamWaitEvent(s, ctx->ev_out[b], 0), "offload wait");
    }
    prof_mark(ctx, slot, 4, s);
    return SCAPE_OK;
}

int dense_common(scape_ctx* ctx, float* x, float* m, float* v, const uint16_t* const* g, void* stream, bool il) {
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    if (!x || !m || !v) return fail(SCAPE_ERR_INVALID_ARG, "x, m and v must not be NULL");
    if (!aligned(x, 16) || !aligned(m, 16) || !aligned(v, 16))
        return fail(SCAPE_ERR_ALIGN, "x, m and v must be 16-byte aligned");
    if (!g) return fail(SCAPE_ERR_INVALID_ARG, "g must not be NULL");
    const int W = ctx->cfg.workers;
    WorkerPtrs wp{};
    wp.ws = il ? 64u * (uint32_t)W : 64u;
    for (int i = 0; i < W; ++i) {
        const uint16_t* gi = il ? g[0] : g[i];
        if (!gi) return fail(SCAPE_ERR_INVALID_ARG, "g[%d] is NULL", il ? 0 : i);
        if (!aligned(gi, 16)) return fail(SCAPE_ERR_ALIGN, "g[%d] must be 16-byte aligned", il ? 0 : i);
        wp.g[i] = il ? gi + 64 * i : gi;
    }
    int rc;
    if ((rc = check_device(ctx))) return rc;
    StepScalars sc;
    sc.beta1 = ctx->cfg.beta1;
    sc.beta2 = ctx->cfg.beta2;
    sc.c1 = 1.0f - ctx->cfg.beta1;
    sc.c2 = 1.0f - ctx->cfg.beta2;
    sc.lr = ctx->cfg.lr;
    sc.eps = ctx->cfg.eps;
    sc.wd = ctx->cfg.weight_decay;
    sc.W = W;
    SCAPE_HIP(launch_dense_adams((hipStream_t)stream, ctx->d_word_info, ctx->n_words, wp, sc, x, m, v),
              "dense_adams");
    return SCAPE_OK;
}

}  // namespace

extern "C" {

int scape_version(int32_t* major, int32_t* minor) {
    if (!major || !minor) return fail(SCAPE_ERR_INVALID_ARG, "NULL output");
    *major = SCAPE_VERSION_MAJOR;
    *minor = SCAPE_VERSION_MINOR;
    return SCAPE_OK;
}

const char* scape_last_error(void) { return g_last_error.c_str(); }

int scape_layout(const scape_config* cfg, int64_t* n_pad, int64_t* k_total, int64_t* layer_offset, int64_t* layer_k,
                 int32_t* layer_owner) {
    int rc = validate_config(cfg);
    if (rc) return rc;
    HostLayout h;
    build_layout(cfg, &h);
    if (n_pad) *n_pad = h.n_pad;
    if (k_total) *k_total = h.k_total;
    for (int32_t l = 0; l < h.L; ++l) {
        if (layer_offset) layer_offset[l] = h.off[l];
        if (layer_k) layer_k[l] = h.k[l];
    }
    if (layer_owner) owner_map(h, cfg->owner_shards ? cfg->owner_shards : cfg->workers, layer_owner);
    return SCAPE_OK;
}

int scape_owner_map(const scape_config* cfg, int32_t num_shards, int32_t* owner) {
    int rc = validate_config(cfg);
    if (rc) return rc;
    if (num_shards < 1) return fail(SCAPE_ERR_INVALID_ARG, "num_shards must be >= 1 (got %d)", num_shards);
    if (!owner) return fail(SCAPE_ERR_INVALID_ARG, "owner is NULL");
    HostLayout h;
    build_layout(cfg, &h);
    owner_map(h, num_shards, owner);
    return SCAPE_OK;
}

int scape_init(const scape_config* cfg, scape_ctx** out) {
    if (!out) return fail(SCAPE_ERR_INVALID_ARG, "out is NULL");
    int rc = validate_config(cfg);
    if (rc) return rc;
    scape_ctx* c = new scape_ctx();
    c->cfg = *cfg;
    c->cfg.layer_numel = nullptr;
    build_layout(cfg, &c->lay);
    c->P = cfg->owner_shards ? cfg->owner_shards : cfg->workers;
    c->owner.resize(c->lay.L);
    owner_map(c->lay, c->P, c->owner.data());
    c->n_words = (uint32_t)(c->lay.n_pad / 64);
    c->n_index_blocks = (c->n_words + kIndexWordsPerBlock - 1) / kIndexWordsPerBlock;


    std::vector<LayerDesc> ld(c->lay.L);
    c->layer_tile0.assign(c->lay.L + 1, 0);
    for (int32_t l = 0; l < c->lay.L; ++l) {
        ld[l].off = (uint32_t)c->lay.off[l];
        ld[l].n = (uint32_t)c->lay.n[l];
        ld[l].k = (uint32_t)c->lay.k[l];
        ld[l].owner = c->owner[l];
        c->layer_tile0[l] = (uint32_t)c->tiles.size();
        const uint32_t w0 = (uint32_t)(c->lay.off[l] / 64);
        const uint32_t w1 = (uint32_t)((c->lay.off[l] + c->lay.n[l] + 63) / 64);
        for (uint32_t w = w0; w < w1; w += kTileWords) {
            TileDesc t;
            t.layer = l;
            t.w0 = w;
            t.w1 = w + kTileWords < w1 ? w + kTileWords : w1;
            t.seg = 0;
            c->tiles.push_back(t);
        }
    }
    c->layer_tile0[c->lay.L] = (uint32_t)c->tiles.size();
    // record segments: runs of kSegTiles tiles inside each layer
    c->layer_seg0.assign(c->lay.L + 1, 0);
    uint64_t rec_total = 0;
    for (int32_t l = 0; l < c->lay.L; ++l) {
        c->layer_seg0[l] = (uint32_t)c->segs.size();
        for (uint32_t t0 = c->layer_tile0[l]; t0 < c->layer_tile0[l + 1]; t0 += kSegTiles) {
            const uint32_t t1 = std::min<uint32_t>(t0 + kSegTiles, c->layer_tile0[l + 1]);
            const uint32_t elems = (c->tiles[t1 - 1].w1 - c->tiles[t0].w0) * 64u;
            SegDesc g;
            g.layer = l;
            g.base = (uint32_t)rec_total;  // below n_pad < 2^31: each space is at most its elements
            g.size = std::min<uint32_t>(elems, (elems >> kRecordShift) + kRecordSlack);
            g.pad = 0;
            rec_total += g.size;
            for (uint32_t t = t0; t < t1; ++t) c->tiles[t].seg = (uint32_t)c->segs.size();
            c->segs.push_back(g);
        }
    }
    c->layer_seg0[c->lay.L] = (uint32_t)c->segs.size();
    const size_t n_segs = c->segs.size();
    // a layer's segments are consecutive in the record buffer: together they
    // are its whole record space
    std::vector<SegDesc> lspace(c->lay.L);
    for (int32_t l = 0; l < c->lay.L; ++l) {
        SegDesc g{};
        g.layer = l;
        for (uint32_t q = c->layer_seg0[l]; q < c->layer_seg0[l + 1]; ++q) {
            if (q == c->layer_seg0[l]) g.base = c->segs[q].base;
            g.size += c->segs[q].size;
        }
        lspace[l] = g;
    }
    c->cand_cap = (uint32_t)rec_total;
    // a segment of s records makes ceil(s / kCandChunk) blocks
    c->vb_cap = (size_t)(rec_total / kCandChunk) + n_segs + 1;
    std::vector<uint16_t> winfo(c->n_words, 0);
    for (int32_t l = 0; l < c->lay.L; ++l) {
        const int64_t off = c->lay.off[l], n = c->lay.n[l];
        for (int64_t w = off / 64; w < (off + n + 63) / 64; ++w) {
            const int64_t inside = std::min<int64_t>(64, off + n - w * 64);
            winfo[w] = (uint16_t)((c->owner[l] << 8) | inside);
        }
    }

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        free_ctx(c);
        return hip_fail(e, "hipGetDevice");
    }
    c->device = dev;
    const size_t L = (size_t)c->lay.L;
    if ((rc = dev_alloc(c, &c->d_layers, L, "layer table")) || (rc = dev_alloc(c, &c->d_tiles, c->tiles.size(), "tile table")) ||
        (rc = dev_alloc(c, &c->d_hist, L * kHistBins, "histograms")) || (rc = dev_alloc(c, &c->d_sel, L, "selection state")) ||
        (rc = dev_alloc(c, &c->d_segs, n_segs, "segment table")) ||
        (rc = dev_alloc(c, &c->d_layer_seg0, L + 1, "layer segment table")) ||
        (rc = dev_alloc(c, &c->d_seg_fill, n_segs, "segment record counters")) ||
        (rc = dev_alloc(c, &c->d_seg_above, n_segs, "segment bit counters")) ||
        (rc = dev_alloc(c, &c->d_lspace, L, "layer record spaces")) ||
        (rc = dev_alloc(c, &c->d_lcount, 3 * L, "layer counters")) ||
        (rc = dev_alloc(c, &c->d_ltick, L, "layer tickets")) ||
        (rc = dev_alloc(c, &c->d_dummy, 4, "load stand-in")) ||
        (rc = dev_alloc(c, &c->d_vb, c->vb_cap, "record blocks")) ||
        (rc = dev_alloc(c, &c->d_vb_count, c->vb_cap, "record block counts")) ||
        (rc = dev_alloc(c, &c->d_totals, 4, "totals")) || (rc = dev_alloc(c, &c->d_miss, 1, "miss flag")) ||
        (rc = dev_alloc(c, &c->d_cand, (size_t)c->cand_cap, "candidate records")) ||
        (rc = dev_alloc(c, &c->d_key16, (size_t)c->lay.n_pad, "statistic keys")) ||
        (rc = dev_alloc(c, &c->d_block_sums,
                        std::max<size_t>((size_t)c->n_index_blocks + 2, ((size_t)c->n_words + kBlock - 1) / kBlock),
                        "index partial sums")) ||
        (rc = dev_alloc(c, &c->d_word_info, (size_t)c->n_words, "word descriptors")) ||
        (rc = dev_alloc(c, &c->d_counts, L, "per-layer counters")) ||
        (rc = dev_alloc(c, &c->d_ovf, L, "per-layer record overflow flags")) ||
        (rc = dev_alloc(c, &c->d_m_stash, (size_t)c->lay.k_total, "m stash")) ||
        (rc = dev_alloc(c, &c->d_union_bits, (size_t)c->n_words, "union staging bits"))) {
        free_ctx(c);
        return rc;
    }
    // the update's stream and its fork/join events (default priority; the events only order work)
    e = hipStreamCreateWithFlags(&c->s_upd, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming);
    if (e != hipSuccess) {
        free_ctx(c);
        return hip_fail(e, "creating the update stream and events");
    }
    e = hipMemcpy(c->d_layers, ld.data(), L * sizeof(LayerDesc), hipMemcpyHostToDevice);
    if (e == hipSuccess && !c->tiles.empty())
        e = hipMemcpy(c->d_tiles, c->tiles.data(), c->tiles.size() * sizeof(TileDesc), hipMemcpyHostToDevice);
    if (e == hipSuccess && n_segs)
        e = hipMemcpy(c->d_segs, c->segs.data(), n_segs * sizeof(SegDesc), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(c->d_lspace, lspace.data(), L * sizeof(SegDesc), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(c->d_lcount, 0, 3 * L * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(c->d_ltick, 0, L * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMemset(c->d_dummy, 0, 4 * sizeof(float));
    if (e == hipSuccess)
        e = hipMemcpy(c->d_layer_seg0, c->layer_seg0.data(), (L + 1) * sizeof(uint32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess && c->n_words)
        e = hipMemcpy(c->d_word_info, winfo.data(), (size_t)c->n_words * sizeof(uint16_t), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(c->d_hist, 0, L * kHistBins * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(c->d_sel, 0, L * sizeof(SelState));
    if (e == hipSuccess) e = hipMemset(c->d_totals, 0, 4 * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(c->d_miss, 0, sizeof(uint32_t));  // no flags before the first selection
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        free_ctx(c);
        return hip_fail(e, "uploading context tables");
    }
    *out = c;
    return SCAPE_OK;
}

int scape_set_select_path(scape_ctx* ctx, int32_t path) {
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    if (path != SCAPE_SELECT_PATH_AUTO && path != SCAPE_SELECT_PATH_SAMPLED && path != SCAPE_SELECT_PATH_COMPACT)
        return fail(SCAPE_ERR_INVALID_ARG, "unknown selection path %d", path);
    ctx->select_path = path;
    return SCAPE_OK;
}

int scape_set_offload_path(scape_ctx* ctx, int32_t path) {
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    if (path != SCAPE_OFFLOAD_PATH_AUTO && path != SCAPE_OFFLOAD_PATH_STAGED)
        return fail(SCAPE_ERR_INVALID_ARG, "unknown offload path %d", path);
    ctx->offload_path = path;
    return SCAPE_OK;
}

int scape_set_update_in_dense_pass(scape_ctx* ctx, int32_t on) {
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    if (on != 0 && on != 1) return fail(SCAPE_ERR_INVALID_ARG, "update_in_dense_pass takes 0 or 1, not %d", on);
    ctx->update_in_dense = on != 0;
    return SCAPE_OK;
}

int scape_workspace_bytes(const scape_ctx* ctx, int64_t* bytes) {
    if (!ctx || !bytes) return fail(SCAPE_ERR_INVALID_ARG, "NULL argument");
    *bytes = (int64_t)ctx->ws_bytes;
    return SCAPE_OK;
}

int scape_selection_flags(scape_ctx* ctx, uint32_t* flags) {
    if (!ctx || !flags) return fail(SCAPE_ERR_INVALID_ARG, "NULL argument");
    int rc;
    if ((rc = check_device(ctx))) return rc;
    uint32_t f = 0;
    SCAPE_HIP(hipMemcpy(&f, ctx->d_miss, sizeof(f), hipMemcpyDeviceToHost), "reading the selection flags");
    *flags = f;
    return SCAPE_OK;
}

int scape_destroy(scape_ctx* ctx) {
    if (!ctx) return SCAPE_OK;
    // wait for the context's own device, free its workspaces there, and leave
    // the caller's current device as it was
    int prev = -1;
    const bool switched = hipGetDevice(&prev) == hipSuccess && prev != ctx->device &&
                          hipSetDevice(ctx->device) == hipSuccess;
    hipDeviceSynchronize();
    free_ctx(ctx);
    if (switched) hipSetDevice(prev);
    return SCAPE_OK;
}

int scape_step(scape_ctx* ctx, float* x, float* m, float* v, float* const* r, const uint16_t* const* g,
               const scape_mask* cur, const scape_mask* next, float* const* sparse_bufs, uint32_t* key_out,
               void* stream) {
    return step_common(ctx, x, m, v, r, g, cur, next, sparse_bufs, key_out, stream, WorkerLayout::kSeparate);
}

int scape_step_interleaved(scape_ctx* ctx, float* xv, float* m, float* r_il, const uint16_t* g_il,
                           const scape_mask* cur, const scape_mask* next, float* const* sparse_bufs, uint32_t* key_out,
                           void* stream) {
    float* r[1] = {r_il};
    const uint16_t* g[1] = {g_il};
    return step_common(ctx, xv, m, nullptr, r, g, cur, next, sparse_bufs, key_out, stream, WorkerLayout::kInterleaved);
}

int scape_step_offload(scape_ctx* ctx, float* x, float* m, float* v, float* const* r_host, const uint16_t* const* g,
                       const scape_mask* cur, const scape_mask* next, float* const* sparse_bufs, uint32_t* key_out,
                       void* stream) {
    return step_common(ctx, x, m, v, r_host, g, cur, next, sparse_bufs, key_out, stream, WorkerLayout::kHostResiduals);
}

int scape_dense_step(scape_ctx* ctx, float* x, float* m, float* v, const uint16_t* const* g, void* stream) {
    return dense_common(ctx, x, m, v, g, stream, false);
}

int scape_dense_step_interleaved(scape_ctx* ctx, float* x, float* m, float* v, const uint16_t* g_il, void* stream) {
    const uint16_t* g[1] = {g_il};
    return dense_common(ctx, x, m, v, g, stream, true);
}

int scape_mask_build(scape_ctx* ctx, const float* mtilde, int32_t num_shards, int32_t shard, const scape_mask* out,
                     void* stream) {
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    if (!mtilde) return fail(SCAPE_ERR_INVALID_ARG, "mtilde is NULL");
    if (!aligned(mtilde, 16)) return fail(SCAPE_ERR_ALIGN, "mtilde must be 16-byte aligned");
    const bool all = num_shards <= 0 || shard < 0;
    if (!all && shard >= num_shards)
        return fail(SCAPE_ERR_INVALID_ARG, "shard %d out of range for %d shards", shard, num_shards);
    int rc;
    if ((rc = check_mask(out, all, "out"))) return rc;
    if ((rc = check_device(ctx))) return rc;
    hipStream_t s = (hipStream_t)stream;
    int32_t la = 0, lb = ctx->lay.L;  // layer range [la, lb)
    if (!all) {
        std::vector<int32_t> own(ctx->lay.L);
        owner_map(ctx->lay, num_shards, own.data());
        la = ctx->lay.L;
        lb = ctx->lay.L;
        for (int32_t l = 0; l < ctx->lay.L; ++l)
            if (own[l] == shard) {
                if (la == ctx->lay.L) la = l;
                lb = l + 1;
            }
        if (la >= lb) return SCAPE_OK;  // the shard owns no layer
    }
    const uint32_t ta = ctx->layer_tile0[la], tb = ctx->layer_tile0[lb];
    const uint32_t wa = (uint32_t)(ctx->lay.off[la] / 64), wb = ctx->layer_tile0[lb] > ctx->layer_tile0[la]
                                                                 ? ctx->tiles[ctx->layer_tile0[lb] - 1].w1
                                                                 : wa;
    SCAPE_HIP(launch_keys_from_mtilde(s, ctx->d_word_info, wa, wb, mtilde, ctx->d_key16), "keys");
    KeySource ks{};
    ks.mtilde = mtilde;
    ZeroRanges rows{};  // the range's histogram rows (the step's dense pass clears them on its way)
    rows.add(ctx->d_hist + (size_t)la * kHistBins, (uint64_t)(lb - la) * kHistBins);
    if ((rc = run_select(ctx, la, lb - la, ta, tb, ctx->d_key16, ks, out->bits, s, nullptr, rows))) return rc;
    if (all && (rc = run_index(ctx, out, s))) return rc;
    return SCAPE_OK;
}

int scape_mask_union_add(scape_ctx* ctx, const float* mtilde, uint64_t* acc_bits, void* stream) {
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    if (!mtilde || !acc_bits) return fail(SCAPE_ERR_INVALID_ARG, "mtilde and acc_bits must not be NULL");
    if (!aligned(mtilde, 16) || !aligned(acc_bits, 16))
        return fail(SCAPE_ERR_ALIGN, "mtilde and acc_bits must be 16-byte aligned");
    int rc;
    if ((rc = check_device(ctx))) return rc;
    hipStream_t s = (hipStream_t)stream;
    const int32_t L = ctx->lay.L;
    if (L == 0 || ctx->tiles.empty()) return SCAPE_OK;
    SCAPE_HIP(launch_keys_from_mtilde(s, ctx->d_word_info, 0, ctx->n_words, mtilde, ctx->d_key16), "keys");
    KeySource ks{};
    ks.mtilde = mtilde;
    ZeroRanges rows{};
    rows.add(ctx->d_hist, (uint64_t)L * kHistBins);
    if ((rc = run_select(ctx, 0, L, 0, (uint32_t)ctx->tiles.size(), ctx->d_key16, ks, ctx->d_union_bits, s, nullptr,
                         rows)))
        return rc;
    SCAPE_HIP(launch_or_words(s, ctx->d_union_bits, acc_bits, ctx->n_words), "or_words");
    return SCAPE_OK;
}

int scape_mask_index(scape_ctx* ctx, const scape_mask* mask, void* stream) {
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    int rc;
    if ((rc = check_mask(mask, true, "mask"))) return rc;
    if ((rc = check_device(ctx))) return rc;
    return run_index(ctx, mask, (hipStream_t)stream);
}

int scape_mask_index_static(const uint64_t* bits, int64_t n_words, uint32_t* idx, int64_t k_cap,
                            uint32_t* block_prefix, void* stream) {
    if (n_words < 0) return fail(SCAPE_ERR_INVALID_ARG, "n_words must be >= 0");
    if (n_words > kIndexStaticMaxWords)
        return fail(SCAPE_ERR_SHAPE, "n_words %lld exceeds the static scratch's maximum of %lld words",
                    (long long)n_words, (long long)kIndexStaticMaxWords);
    if (k_cap < 0 || k_cap > (int64_t)0xFFFFFFFFu) return fail(SCAPE_ERR_INVALID_ARG, "k_cap must be in 0..2^32-1");
    if (!bits || !block_prefix || (k_cap > 0 && !idx))
        return fail(SCAPE_ERR_INVALID_ARG, "bits, block_prefix and (for k_cap > 0) idx must not be NULL");
    if (!aligned(bits, 8)) return fail(SCAPE_ERR_ALIGN, "bits must be 8-byte aligned");
    if (!aligned(block_prefix, 4) || (idx && !aligned(idx, 4)))
        return fail(SCAPE_ERR_ALIGN, "idx and block_prefix must be 4-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const uint32_t nw = (uint32_t)n_words;
    if (nw == 0) {  // an empty mask: the prefix is the one total, 0
        SCAPE_HIP(launch_fill_u32(s, block_prefix, 1, 0u), "fill");
        return SCAPE_OK;
    }
    uint32_t* scratch = nullptr;
    SCAPE_HIP(index_scratch(&scratch), "index scratch address");
    SCAPE_HIP(launch_index_count(s, bits, nw, scratch), "index_count");
    SCAPE_HIP(launch_index_scan(s, scratch, (nw + kIndexWordsPerBlock - 1) / kIndexWordsPerBlock), "index_scan");
    SCAPE_HIP(launch_index_emit(s, bits, nw, scratch, idx, (uint32_t)k_cap, block_prefix), "index_emit");
    return SCAPE_OK;
}

int scape_pack(const uint8_t* pred, int64_t n, uint64_t* bits, void* stream) {
    if (n < 0) return fail(SCAPE_ERR_INVALID_ARG, "n must be >= 0");
    if (n >= (int64_t(1) << 37)) return fail(SCAPE_ERR_SHAPE, "n too large");
    if (n == 0) return SCAPE_OK;
    if (!pred || !bits) return fail(SCAPE_ERR_INVALID_ARG, "pred and bits must not be NULL");
    if (!aligned(bits, 8)) return fail(SCAPE_ERR_ALIGN, "bits must be 8-byte aligned");
    SCAPE_HIP(launch_pack((hipStream_t)stream, pred, n, bits), "pack");
    return SCAPE_OK;
}

int scape_unpack(const uint64_t* bits, int64_t n, uint8_t* pred, void* stream) {
    if (n < 0) return fail(SCAPE_ERR_INVALID_ARG, "n must be >= 0");
    if (n >= (int64_t(1) << 37)) return fail(SCAPE_ERR_SHAPE, "n too large");
    if (n == 0) return SCAPE_OK;
    if (!pred || !bits) return fail(SCAPE_ERR_INVALID_ARG, "pred and bits must not be NULL");
    if (!aligned(bits, 8)) return fail(SCAPE_ERR_ALIGN, "bits must be 8-byte aligned");
    SCAPE_HIP(launch_unpack((hipStream_t)stream, bits, n, pred), "unpack");
    return SCAPE_OK;
}

int scape_copy_probe(const void* src, void* dst, uint64_t bytes, void* stream) {
    if (bytes == 0) return SCAPE_OK;
    if (!src || !dst) return fail(SCAPE_ERR_INVALID_ARG, "src and dst must not be NULL");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(SCAPE_ERR_ALIGN, "src and dst must be 16-byte aligned");
    if (bytes % 16 != 0) return fail(SCAPE_ERR_SHAPE, "bytes must be a multiple of 16");
    if (bytes / 16 > (uint64_t)0xFFFFFFFFu * kBlock) return fail(SCAPE_ERR_SHAPE, "bytes too large");
    SCAPE_HIP(launch_copy_probe((hipStream_t)stream, src, dst, bytes / 16), "copy_probe");
    return SCAPE_OK;
}

int scape_stream_probe(const void* const* src, const uint32_t* src_width, int32_t n_src, void* const* dst,
                       const uint32_t* dst_width, int32_t n_dst, uint64_t n_words, void* stream) {
    if (n_src < 0 || n_src > kStreamProbeMax || n_dst < 0 || n_dst > kStreamProbeMax || n_src + n_dst == 0)
        return fail(SCAPE_ERR_INVALID_ARG, "n_src and n_dst must be 0..%d, not both 0", kStreamProbeMax);
    if ((n_src && (!src || !src_width)) || (n_dst && (!dst || !dst_width)))
        return fail(SCAPE_ERR_INVALID_ARG, "array lists must not be NULL");
    if (n_words > 0xFFFFFFFFull - kWaves) return fail(SCAPE_ERR_SHAPE, "n_words too large");
    StreamProbe a{};
    a.n_src = n_src;
    a.n_dst = n_dst;
    auto ok_width = [](uint32_t w) { return w == 2 || w == 4 || w == 8 || w == 16; };
    for (int i = 0; i < n_src; ++i) {
        if (!src[i]) return fail(SCAPE_ERR_INVALID_ARG, "src[%d] is NULL", i);
        if (!ok_width(src_width[i])) return fail(SCAPE_ERR_INVALID_ARG, "src_width[%d] must be 2, 4, 8 or 16", i);
        if (!aligned(src[i], src_width[i])) return fail(SCAPE_ERR_ALIGN, "src[%d] must be aligned to its width", i);
        a.src[i] = static_cast<const uint8_t*>(src[i]);
        a.src_width[i] = src_width[i];
    }
    for (int i = 0; i < n_dst; ++i) {
        if (!dst[i]) return fail(SCAPE_ERR_INVALID_ARG, "dst[%d] is NULL", i);
        if (!ok_width(dst_width[i])) return fail(SCAPE_ERR_INVALID_ARG, "dst_width[%d] must be 2, 4, 8 or 16", i);
        if (!aligned(dst[i], dst_width[i])) return fail(SCAPE_ERR_ALIGN, "dst[%d] must be aligned to its width", i);
        a.dst[i] = static_cast<uint8_t*>(dst[i]);
        a.dst_width[i] = dst_width[i];
    }
    SCAPE_HIP(launch_stream_probe((hipStream_t)stream, a, (uint32_t)n_words), "stream_probe");
    return SCAPE_OK;
}

int scape_reduce_sparse(const float* const* bufs, int32_t W, int64_t k, float* out, void* stream) {
    if (W < 1 || W > SCAPE_MAX_WORKERS) return fail(SCAPE_ERR_INVALID_ARG, "W must be in 1..%d", SCAPE_MAX_WORKERS);
    if (k < 0) return fail(SCAPE_ERR_INVALID_ARG, "k must be >= 0");
    if (k >= kMaxFlat * 4) return fail(SCAPE_ERR_SHAPE, "k too large");
    if (k == 0) return SCAPE_OK;
    if (!bufs || !out) return fail(SCAPE_ERR_INVALID_ARG, "bufs and out must not be NULL");
    for (int i = 0; i < W; ++i) {
        if (!bufs[i]) return fail(SCAPE_ERR_INVALID_ARG, "bufs[%d] is NULL", i);
        if (!aligned(bufs[i], 4)) return fail(SCAPE_ERR_ALIGN, "bufs[%d] must be 4-byte aligned", i);
    }
    if (!aligned(out, 4)) return fail(SCAPE_ERR_ALIGN, "out must be 4-byte aligned");
    SCAPE_HIP(launch_reduce_sparse((hipStream_t)stream, bufs, W, k, out), "reduce_sparse");
    return SCAPE_OK;
}

int scape_profile_enable(scape_ctx* ctx, int32_t enable) {
    if (!ctx) return fail(SCAPE_ERR_INVALID_ARG, "ctx is NULL");
    if (enable && !ctx->prof_events) {
        for (auto& s : ctx->prof)
            for (auto& e : s.ev) SCAPE_HIP(hipEventCreate(&e), "hipEventCreate");
        ctx->prof_events = true;
    }
    if (enable) {
        for (auto& s : ctx->prof) s.pending = false;
        for (double& d : ctx->prof_ms) d = 0.0;
        ctx->prof_steps = 0;
        ctx->prof_next = 0;
    }
    ctx->prof_on = enable != 0;
    return SCAPE_OK;
}

int scape_profile_read(scape_ctx* ctx, double* ms, int64_t* steps) {
    if (!ctx || !ms || !steps) return fail(SCAPE_ERR_INVALID_ARG, "NULL argument");
    for (int i = 0; i < kProfSlots; ++i) prof_collect(ctx, (ctx->prof_next + i) % kProfSlots);
    for (int i = 0; i < SCAPE_PHASE_COUNT; ++i) ms[i] = ctx->prof_ms[i];
    *steps = ctx->prof_steps;
    return SCAPE_OK;
}

}  // extern "C"
