// scape_internal.h - types shared by the host orchestration (scape_api.cpp)
// and the gfx950 kernels (k_*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scape.h"

namespace scape {

// ---------------------------------------------------------------------------
// Launch geometry.  A "tile" is a run of whole 64-element words inside one
// layer; the key-sampling and filter kernels give one tile to a workgroup.
constexpr int kBlock = 256;             // threads per workgroup (4 waves of 64)
constexpr int kWaves = kBlock / 64;
#ifndef SCAPE_TILE_WORDS
#define SCAPE_TILE_WORDS 512
#endif
constexpr int kTileWords = SCAPE_TILE_WORDS;  // words per tile (512 words = 32768 elements)
// Radix digits of the 31-bit key: the first digit is bits 30..18 (8
// exponent bits and 5 mantissa bits: buckets of 1/32 octave), then key bits
// 17..15, 14..6 and 5..0; ties are split on the layer position, bits 30..20,
// 19..10 and 9..0.  The stored keys are bits 30..15, so the first two digits
// need no full key.
constexpr int kDigit1Bits = 13;
constexpr int kDigit1Shift = 31 - kDigit1Bits;  // 18
constexpr int kDigit1Bins = 1 << kDigit1Bits;   // 8192
constexpr int kKeyShift = 15;                   // a 16-bit stored key is bits 30..15 of the 31-bit key
constexpr int kDigit1FromKey16 = kDigit1Shift - kKeyShift;  // first digit = stored 16-bit key >> 3
constexpr int kKey2Bits = kDigit1Shift - kKeyShift;         // 3: bits 17..15
constexpr int kKey3Bits = 9;                                // bits 14..6
constexpr int kKey4Bits = kKeyShift - kKey3Bits;            // 6: bits 5..0
constexpr int kHistBins = kDigit1Bins;          // histogram row per layer (>= every digit's bins)
constexpr int kIndexWordsPerBlock = 2048;  // words per workgroup in the index passes
constexpr uint32_t kIndexSmallMaxWords = (uint32_t)kBlock * kBlock;  // masks indexed in two launches
// Largest word count of the context-free index (every layout the ABI takes:
// n_pad < 2^31 elements), and the entries of its static partial-sum array
// (one per index workgroup, plus the total).
constexpr int64_t kIndexStaticMaxWords = int64_t(1) << 25;
constexpr int kIndexScratchEntries = (int)(kIndexStaticMaxWords / kIndexWordsPerBlock) + 2;
// The compact selection path takes a range whose layers all hold at most
// kCompactMaxLayer elements (one workgroup finishes each layer); its two
// launches split tiles until they have about kCompact*Blocks workgroups.
#ifndef SCAPE_COMPACT_MAX_LAYER
#define SCAPE_COMPACT_MAX_LAYER (1 << 22)
#endif
constexpr int64_t kCompactMaxLayer = SCAPE_COMPACT_MAX_LAYER;
constexpr uint32_t kCompactHistBlocks = 128, kCompactHistParts = 4;
constexpr uint32_t kCompactFilterBlocks = 256, kCompactFilterParts = 4;
constexpr int kCandChunk = 8192;        // candidate records per virtual block
constexpr int kSegTiles = 16;           // tiles per record segment

struct TileDesc {
    int32_t layer;
    uint32_t w0;   // first word
    uint32_t w1;   // one past the last word
    uint32_t seg;  // record segment holding this tile's records
};

// A record segment: up to kSegTiles consecutive tiles of one layer.  Their
// candidate records go to the segment's own range of the record buffer,
// [base, base + size): the workgroups in flight at one time reserve space on
// many different counters instead of one per layer.  The range holds a
// fraction of the segment's elements (the record space); records past it are
// dropped and counted, and the layer is then redone exactly.
struct SegDesc {
    int32_t layer;
    uint32_t base;  // first record slot
    uint32_t size;  // record slots
    uint32_t pad;
};
// Record space of a segment of e elements: e / 2^kRecordShift + kRecordSlack
// slots (at most e).  Windows from the sampled histogram hold 1-3% of a
// layer's keys on the workloads measured.
constexpr int kRecordShift = 4;
constexpr uint32_t kRecordSlack = 1024;

struct LayerDesc {
    uint32_t off;    // first element (multiple of 64)
    uint32_t n;      // elements
    uint32_t k;      // kept count (<= n)
    int32_t owner;   // worker whose candidate is the statistic
};

// Per-layer state of the radix selection.  The final rule for a layer is
//   selected(j) = !none && (key > T || (key == T && jl <= J))
// where jl is the layer-local position.
enum SelPhase : uint32_t {
    kPhaseDone = 0,
    kPhaseKey2 = 1,   // key bits 17..15 pending
    kPhaseKey3 = 2,   // key bits 14..6 pending (its pass fetches the full keys)
    kPhaseKey4 = 3,   // key bits 5..0 pending
    kPhasePos1 = 4,   // tie position bits 30..20 pending
    kPhasePos2 = 5,   // tie position bits 19..10 pending
    kPhasePos3 = 6,   // tie position bits 9..0 pending
};

struct SelState {
    uint32_t phase;
    uint32_t none;        // layer selects nothing (k == 0 or not built)
    uint32_t all_bucket;  // whole first-digit bucket taken: no candidates
    uint32_t d1;          // first-digit bucket of the threshold
    uint32_t need;        // still to take among records matching the prefix
    uint32_t kprefix;     // resolved high bits of T
    uint32_t jprefix;     // resolved high bits of J
    uint32_t T;
    uint32_t J;
    uint32_t n_lo, n_hi;  // first-digit window the filter made records for (n_lo > n_hi: none)
    uint32_t mode;        // 0 decided by the window, 1 reclassified, 2 full histogram needed
    uint32_t pad[6];
};

// A block of at most kCandChunk candidate records of one layer.
struct VblockDesc {
    uint32_t p0;  // first record
    int32_t layer;
};

// Worker i's residual and gradient of element j = 64 w + l (l < 64) are
// r[i][w * ws + l] and g[i][w * ws + l]: ws = 64 for one array per worker,
// ws = 64 W for the worker-interleaved layout, where each 64-element word
// holds the W workers' 64 values one after another (r[i] = base + 64 i).
struct WorkerPtrs {
    float* r[SCAPE_MAX_WORKERS];
    const uint16_t* g[SCAPE_MAX_WORKERS];
    float* b[SCAPE_MAX_WORKERS];
    uint32_t ws;
};

// Where the selection finds the full 31-bit key of a candidate (the stored
// keys keep only their top 16 bits):
//   mtilde != nullptr: the magnitude bits of mtilde[j];
//   else key32 != nullptr: key32[j];
//   else recomputed from the step's state: on the current mask (rank below
//   k_cap) the owner's sparse buffer entry, off it beta1*m[j] + c1*r_owner[j]
//   (m is unchanged and r holds the error-compensated gradient there), the
//   same fp32 operations in the same order as the dense pass.
struct KeySource {
    const float* mtilde;
    const uint32_t* key32;
    const float* m;
    const float* r[SCAPE_MAX_WORKERS];  // word stride ws, as in WorkerPtrs
    uint32_t ws;
    const float* b[SCAPE_MAX_WORKERS];
    const uint64_t* cur_bits;
    const uint32_t* cur_prefix;
    uint32_t k_cap;
    float beta1, c1;
};

struct StepScalars {
    float beta1, beta2, c1, c2, lr, eps, wd;
    int32_t W;
};

// ---------------------------------------------------------------------------
// Kernel launchers (k_*.hip).  Each returns the hipError_t of the launch.

// elementwise: error feedback, candidates, compaction, statistic, digit-1
// histogram; then reduction + reconstruction + update.
// clear[0, n_clear) is zeroed on the way (the selection's histogram rows).
// upd 0: the update is left to launch_reduce_update (m_stash written);
// upd 1 / 2: the pass also updates m, v, x at the mask's positions (x and v
// apart / x holding (x, v) pairs), touching them there only; `dummy` is 8
// bytes nothing writes.  upd 3 / 4: the same, streaming x, v and m whole
// (upd 4: the (x, v) pairs of lines that hold a masked element) and storing
// the unmasked elements' old values back.
hipError_t launch_ef_compact(hipStream_t s, const uint16_t* word_info, uint32_t n_words, const WorkerPtrs& wp,
                             const StepScalars& sc, float* m, const uint64_t* cur_bits,
                             const uint32_t* cur_prefix, uint32_t k_cap, uint16_t* key16, uint32_t* key32,
                             float* m_stash, uint32_t* clear, uint32_t n_clear, int upd, float* x, float* v,
                             const float* dummy);
// xv_pairs: x is an array of (x, v) pairs (x at 2j, v at 2j + 1) and v is
// not used.
hipError_t launch_reduce_update(hipStream_t s, const WorkerPtrs& wp, const StepScalars& sc, float* x, float* m,
                                float* v, bool xv_pairs, const uint32_t* cur_idx, const uint32_t* cur_prefix,
                                const float* m_stash, uint32_t n_words, uint32_t n_pad, uint32_t k_cap);
hipError_t launch_dense_adams(hipStream_t s, const uint16_t* word_info, uint32_t n_words, const WorkerPtrs& wp,
                              const StepScalars& sc, float* x, float* m, float* v);
hipError_t launch_keys_from_mtilde(hipStream_t s, const uint16_t* word_info, uint32_t w_begin, uint32_t w_end,
                                   const float* mtilde, uint16_t* key16);
hipError_t launch_reduce_sparse(hipStream_t s, const float* const* bufs, int32_t W, int64_t k, float* out);
hipError_t launch_fill_u32(hipStream_t s, uint32_t* p, uint64_t n, uint32_t value);
// Up to kZeroRangesMax arrays of 32-bit words zeroed by one launch (ranges of
// n = 0 are allowed; nothing is launched if every range is empty).  add()
// does not check the count: the selection adds four ranges to at most two
// of its caller's.
constexpr int kZeroRangesMax = 6;
struct ZeroRanges {
    uint32_t* p[kZeroRangesMax];
    uint64_t n[kZeroRangesMax];
    int32_t count;
    void add(uint32_t* ptr, uint64_t words) {
        p[count] = ptr;
        n[count] = words;
        ++count;
    }
};
hipError_t launch_zero_ranges(hipStream_t s, const ZeroRanges& zr);

// selection
hipError_t launch_sample_hist(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                              const uint16_t* key, uint32_t* hist, uint32_t* sample_count);
hipError_t launch_estimate(hipStream_t s, int32_t layer0, int32_t n_layers, const LayerDesc* layers, uint32_t* hist,
                           const uint32_t* sample_count, SelState* st, uint32_t* miss);
// `miss` is one word: k_estimate clears it, k_select_first sets it when a
// layer's threshold falls outside its window, and the fallback kernels
// (k_hist_full, k_filter_exact) return at once while it is clear.
// Record segments: `segs`, `seg_fill` (records per segment) and `seg_above`
// (keys above the window per segment) are indexed by global segment number.
// The filter also counts its records' first digits into each layer's
// histogram row (hist, kHistBins per layer), for k_select_first.
hipError_t launch_filter(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                         const SegDesc* segs, const SelState* st, const uint16_t* key, uint64_t* bits,
                         uint32_t* seg_fill, uint64_t* cand, uint32_t* seg_above, uint32_t* hist);
// ovf[l] != 0: layer l lost records to its record space in the key filter.
hipError_t launch_select_first(hipStream_t s, int32_t layer0, int32_t n_layers, bool first_pass,
                               const LayerDesc* layers, const uint32_t* layer_seg0, uint32_t* hist, SelState* st,
                               const uint32_t* seg_above, uint32_t* seg_fill, const uint32_t* ovf, uint32_t* miss);
hipError_t launch_hist_full(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                            const SelState* st, const uint16_t* key, uint32_t* hist, const uint32_t* miss);
hipError_t launch_filter_exact(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, const LayerDesc* layers,
                               const SegDesc* segs, const SelState* st, const uint16_t* key, uint64_t* bits,
                               uint32_t* seg_fill, uint64_t* cand, uint32_t* seg_above, const uint32_t* miss);
hipError_t launch_cand_scan(hipStream_t s, uint32_t seg0, uint32_t n_segs, const SegDesc* segs,
                            const uint32_t* seg_fill, VblockDesc* vb, uint32_t* vb_count, uint32_t* totals,
                            bool second, uint32_t* ovf, SelState* st, uint32_t* miss);

// A record pass also runs the same phase over the keys of the layers that
// lost records even in their exact bucket (bit 1 of *miss), walking tiles.
hipError_t launch_cand_pass(hipStream_t s, uint32_t phase, const VblockDesc* vb, uint32_t* vb_count,
                            const uint32_t* totals, const LayerDesc* layers, const SelState* st,
                            const KeySource& ks, uint64_t* cand, uint32_t* hist, uint64_t* bits,
                            const TileDesc* tiles, uint32_t n_tiles, const uint16_t* key, const uint32_t* miss);
hipError_t launch_select_next(hipStream_t s, uint32_t phase, int32_t layer0, int32_t n_layers, uint32_t* hist,
                              SelState* st);

// The compact path (every layer of the range small): tiles split over
// `parts` workgroups each.  Per layer: lspace[l] its whole record space,
// ticket[l] the workgroups' ticket counter (zero between launches; 64-bit
// for the filter, whose low half also sums the records), lrec[l] and
// labove[l] its record and bit counters.  k_compact_hist leaves every
// layer of the range with its exact threshold bucket in st; k_compact_filter
// writes the layers' mask words and finishes them.
hipError_t launch_compact_hist(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, uint32_t parts,
                               const LayerDesc* layers, const uint16_t* key, uint32_t* hist, SelState* st,
                               uint32_t* ticket, uint32_t* lrec, uint32_t* labove, uint32_t* miss);
hipError_t launch_compact_filter(hipStream_t s, const TileDesc* tiles, uint32_t n_tiles, uint32_t parts,
                                 const LayerDesc* layers, const SegDesc* lspace, SelState* st, const uint16_t* key,
                                 const KeySource& ks, uint64_t* bits, uint64_t* cand, unsigned long long* ticket,
                                 uint32_t* lrec, uint32_t* labove, uint32_t* miss);

// bits
hipError_t launch_index_count(hipStream_t s, const uint64_t* bits, uint32_t n_words, uint32_t* block_sums);
hipError_t launch_index_scan(hipStream_t s, uint32_t* block_sums, uint32_t n_blocks);
hipError_t launch_index_emit(hipStream_t s, const uint64_t* bits, uint32_t n_words, const uint32_t* block_offs,
                             uint32_t* idx, uint32_t k_cap, uint32_t* prefix);
// Both index launches for a mask of at most kIndexSmallMaxWords words
// (block_sums: one entry per kBlock words).
hipError_t launch_index_small(hipStream_t s, const uint64_t* bits, uint32_t n_words, uint32_t* block_sums,
                              uint32_t* idx, uint32_t k_cap, uint32_t* prefix);
// Device address (on the current device) of the index's file-scope
// partial-sum array, looked up once per device.
hipError_t index_scratch(uint32_t** out);
hipError_t launch_or_words(hipStream_t s, const uint64_t* src, uint64_t* acc, uint32_t n_words);
hipError_t launch_pack(hipStream_t s, const uint8_t* pred, int64_t n, uint64_t* bits);
hipError_t launch_unpack(hipStream_t s, const uint64_t* bits, int64_t n, uint8_t* pred);
hipError_t launch_copy_probe(hipStream_t s, const void* src, void* dst, uint64_t n16);
// A pass that reads n_src arrays and writes n_dst arrays word by word,
// width bytes per lane each (2, 4, 8 or 16), and does nothing else.
constexpr int kStreamProbeMax = 4;
struct StreamProbe {
    const uint8_t* src[kStreamProbeMax];
    uint8_t* dst[kStreamProbeMax];
    uint32_t src_width[kStreamProbeMax], dst_width[kStreamProbeMax];
    int32_t n_src, n_dst;
};
hipError_t launch_stream_probe(hipStream_t s, const StreamProbe& a, uint32_t n_words);

}  // namespace scape
