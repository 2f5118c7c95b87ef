// Internal interface between the host API (tsw_api.cpp) and the gfx950
// kernels (tsw_kernels.hip, tsw_mfma*.hip, tsw_accept.hip).  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsw {

// How the split kernels find a key's K/V row: the cache position itself
// (contiguous), through an index list (gather, the draft pass), through a
// per-sequence block table into a page pool (paged batch), or through both
// (paged draft pass: index list -> position -> page).  kModeContigRoot is the
// contiguous layout that also writes the root row's scores (SplitArgs::root_s).
enum { kModeContig = 0, kModeGather = 1, kModePaged = 2, kModeContigRoot = 3, kModePagedGather = 4 };

// Everything a split kernel needs, passed by value as the kernel argument.
// The tree mask travels here (one 64-bit word per node) so that no device
// buffer or host-to-device copy is needed for it.
struct SplitArgs {
    const void* q;           // [T][Hq][d]
    const void* k;           // [Hkv][rows][d], kv_head_stride elements per head
    const void* v;
    const int32_t* idx;      // partial variant: sorted prefix positions; nullptr for verify
                             // (paged draft pass: sequence b's list at idx + b * idx_stride)
    float* part_o;           // [n_splits][T][Hq][d]
    float* part_lse;         // [n_splits][T][Hq], natural log
    int64_t n_prefix;        // the tree rows start at this cache position
    int64_t kv_head_stride;  // elements
    int64_t n_keys;          // prefix keys in the list: n_prefix (verify) or n_idx (partial)
    int64_t chunk_keys;      // prefix keys per split, a multiple of the kernel's key tile
    int32_t T, Hq, Hkv, G, M, n_splits;
    float scale_log2;        // scale * log2(e): scores are exponentiated base 2
    int32_t B;               // sequences; 1 unless paged (grid x then enumerates every sequence's splits)
    uint64_t mask[64];       // ancestor-or-self bits per node
    // paged batch: k/v point at page pools [n_pages][Hkv][page_rows][d];
    // sequence b's logical page j is table[b * table_stride + j]
    const int32_t* table;
    int32_t table_stride, page_rows, page_shift, pad_;
    int64_t page_bytes;      // Hkv * page_rows * d * 2: one page of the pool
    int64_t npb[64];         // committed length per sequence
    int64_t nib[64];         // paged draft pass: index-list length per sequence
    int64_t idx_stride;      // paged draft pass: entries between sequences' index lists
    // splits of sequence b are grid x in [seg_base[b], seg_base[b+1]), each
    // ceil(n / splits) keys rounded up to whole tiles, but the last
    int32_t seg_base[65];
    // kModeContigRoot (Hq / Hkv <= 16): root_s[h * root_stride + p] =
    // dot(q[0][h], k[g(h)][p]) (unscaled) for every committed position
    // p < n_prefix
    float* root_s;
    int64_t root_stride;     // a multiple of 4
    uint32_t* root_clear;    // kModeContigRoot: 1024 words zeroed by work-group (0, 0), or nullptr
};
// kernel arguments are limited to 4 KB
static_assert(sizeof(SplitArgs) <= 4096, "SplitArgs must fit the kernel-argument segment");

// Partial rows grouped by sequence for the merge: sequence s owns splits
// [base[s], base[s+1]), each split holding rows_per_seg rows.  A single
// sequence has base = {0, n_splits}, rows_per_seg = all rows.
struct MergeSegs {
    int32_t n_seg;
    int32_t pad_;
    int64_t rows_per_seg;    // < 2^31 when n_seg > 1 (T * Hq rows)
    int32_t base[65];
};

// Matrix-core kernel shapes.  A work-group holds `waves` wavefronts: `rgroups`
// groups of query-row blocks (16 rows each, at most `nb` blocks per wave)
// times waves/rgroups sub-tiles of 32 keys per key tile.
struct MfmaConfig {
    int waves, rgroups, nb;
    int tile_keys() const { return 32 * (waves / rgroups); }
};

// Largest index-list slice one work-group stages in LDS (gather variant).
constexpr int kGatherChunkMax = 4096;

// Largest prefix slice of one work-group in the contiguous layout: its K and
// V rows are read through buffer resources with 32-bit byte offsets from the
// slice's first row (256-byte rows, plus the tree rows in the last split).
constexpr int64_t kContigChunkMax = (int64_t)1 << 23;

// Picks the matrix-core shape for M query rows per kv head; returns false
// when no shape covers M (callers then use the vector-ALU kernel).
bool mfma_config_for(int M, MfmaConfig* cfg);

hipError_t launch_split_mfma(const MfmaConfig& cfg, int mode, const SplitArgs& a,
                             int n_kv_heads, hipStream_t stream);
hipError_t launch_split_valu(int dtype, int d, bool gather, const SplitArgs& a, int n_kv_heads,
                             hipStream_t stream);
hipError_t launch_lse_merge(int n_splits, int64_t n_rows, int d, const float* part_o,
                            const float* part_lse, float* o, float* lse, hipStream_t stream);
hipError_t launch_lse_merge_segs(const MergeSegs& segs, int64_t n_rows, const float* part_o,
                                 const float* part_lse, float* o, float* lse, hipStream_t stream);

// Greedy acceptance: per-slice maxima of one node's logits, the tree with
// depths and ancestor-or-self bits (in the kernel arguments, like the mask
// above) and the slice count.
struct AcceptPartial {
    float v;
    int32_t i;
};
struct AcceptArgs {
    int32_t T, n_chunks;
    int32_t parent[64];
    int32_t depth[64];
    uint64_t mask[64];       // ancestor-or-self bits per node
    // contextual penalty folded into the argmax (window > 0)
    int32_t window;
    float theta;
    int64_t n_recent;
    const int32_t* recent;
};
// Largest logit slice of one argmax work-group (its penalty bitmap in LDS).
constexpr int64_t kAcceptSliceMax = 65536;
// Accepted-path compaction of one cache (n_layers x Hkv heads of K and V).
struct CompactArgs {
    void* k;
    void* v;
    int64_t layer_stride;    // elements between layers
    int64_t kv_head_stride;  // elements between kv heads
    int64_t n_prefix;        // tree node j sits at row n_prefix + j
    int32_t T, esz, row_bytes;
};
hipError_t launch_accept(const AcceptArgs& a, const void* logits, int logits_dtype, int64_t vocab, int64_t chunk,
                         bool vec_ok, const int32_t* draft, int32_t* result, AcceptPartial* part,
                         hipStream_t stream);
hipError_t launch_kv_compact(const CompactArgs& a, int n_layers, int n_kv_heads, const int32_t* result,
                             hipStream_t stream);

// Contextual penalty on every node's logits (in place).
constexpr int kPenaltyMaxWindow = 8192;
struct PenaltyArgs {
    int32_t T, window;
    int64_t vocab, n_recent;
    float theta;
    int32_t parent[64];
};
hipError_t launch_context_penalty(const PenaltyArgs& a, void* logits, int logits_dtype, const int32_t* draft,
                                  const int32_t* recent, hipStream_t stream);

// Importance of committed positions (node 0's attention mass) and the
// draft pass's index selection.
constexpr int kSelectChunk = 256;      // keys per importance work-group
constexpr int kSelectMaxHeads = 64;    // query heads held in LDS
struct SelectArgs {
    const void* q;           // [T][Hq][d]; node 0's row is used
    const void* k;           // [Hkv][rows][d]
    const float* lse;        // [T][Hq]; node 0's row is used
    int64_t n_prefix, kv_head_stride;
    int32_t Hq, Hkv, G, d, dtype;
    float scale;
};
// cus: the device's compute units (the key chunks are sized to two work-groups per CU)
hipError_t launch_importance(const SelectArgs& a, float* imp, int cus, hipStream_t stream);
constexpr int64_t kSelBlock = 4096;    // candidates per selection work-group
size_t select_scratch_bytes(int64_t n_prefix);
hipError_t launch_select(const float* imp, int64_t n_prefix, int64_t n_keep, int64_t n_out, int32_t* idx,
                         uint32_t* scratch, hipStream_t stream);
hipError_t launch_select_keep(int64_t n_keep, int32_t* idx, uint32_t* scratch, hipStream_t stream);
// passes first_pass..3 (the earlier passes' totals already in scratch), flags, write
hipError_t launch_select_passes(const float* imp, int64_t n_prefix, int64_t n_keep, int64_t n_out, int32_t* idx,
                                uint32_t* scratch, int first_pass, hipStream_t stream);
// Writes imp and idx[0..n_keep); totals: nullptr, or the scratch's digit
// totals (already zero) to count the first pass's candidates p >= n_keep into
hipError_t launch_importance_from_scores(const float* root_s, int64_t stride, const float* lse, int Hq,
                                         int64_t n_prefix, float c, int64_t n_keep, float* imp, uint32_t* totals,
                                         int32_t* idx, hipStream_t stream);

// Read-stream ceiling (measurement aid): rows [0, rows) of n_kv_heads heads
// of K and V (256-byte rows, head_bytes apart) through the LDS-DMA ring.
hipError_t launch_read_stream(const void* k, const void* v, int n_kv_heads, int64_t head_bytes, int64_t rows,
                              int n_splits, unsigned* sink, hipStream_t stream);

// Launch floor (measurement aid): an empty kernel on a split kernel's grid
// (a.n_splits x n_kv_heads) with `threads` per work-group and a's size of
// by-value arguments.
hipError_t launch_launch_floor(const SplitArgs& a, int n_kv_heads, int threads, hipStream_t stream);

// Key tile of the vector-ALU kernel and its query rows per work-group.
constexpr int kValuTile = 64;
constexpr int kValuRows = 16;

}  // namespace tsw
