// Host side of the tree-verification attention library: argument checks,
// the tree mask builder, the split planner and the C entry points declared
// in include/tsw.h.  Kernels live in tsw_kernels.hip, tsw_mfma*.hip and
// tsw_accept.hip.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "tsw.h"
#include "tsw_internal.h"

namespace {

using tsw::SplitArgs;

constexpr int kMaxNodes = 64;
constexpr float kLog2e = 1.44269504088896340736f;

// Parent encoding of the candidate tree: a single root at index 0
// (parent -1), every other node names an earlier node.  A breadth-first
// numbering of the 3-ary draft tree ("From Hours to Minutes ..." arxivlens
// summary, Technical Contribution) satisfies this, as does any topological
// order.
int build_mask(const int32_t* parent, int32_t T, uint64_t* mask, int32_t* depth) {
    if (!parent || !mask) return TSW_EINVAL;
    if (T < 1 || T > kMaxNodes) return TSW_EINVAL;
    if (parent[0] != -1) return TSW_EBADTREE;
    for (int32_t i = 1; i < T; ++i)
        if (parent[i] < 0 || parent[i] >= i) return TSW_EBADTREE;
    // Parents precede children, so one forward pass extends each parent's
    // ancestor-or-self set by the node itself.
    mask[0] = 1ull;
    if (depth) depth[0] = 0;
    for (int32_t i = 1; i < T; ++i) {
        mask[i] = mask[parent[i]] | (1ull << i);
        if (depth) depth[i] = depth[parent[i]] + 1;
    }
    return TSW_OK;
}

int check_desc(const tsw_attn_desc* d) {
    if (!d) return TSW_EINVAL;
    if (d->reserved != 0) return TSW_EINVAL;
    if (d->T < 1 || d->T > kMaxNodes) return TSW_EINVAL;
    if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv != 0) return TSW_EINVAL;
    if (d->n_prefix < 0) return TSW_EINVAL;
    if (!(d->scale > 0.0f) || !isfinite(d->scale)) return TSW_EINVAL;
    if (d->d != 64 && d->d != 128) return TSW_EUNSUPPORTED;
    if (d->dtype != TSW_DTYPE_F32 && d->dtype != TSW_DTYPE_BF16) return TSW_EUNSUPPORTED;
    if (d->impl != TSW_IMPL_AUTO && d->impl != TSW_IMPL_VALU && d->impl != TSW_IMPL_MFMA) return TSW_EUNSUPPORTED;
    if (d->kv_head_stride < (d->n_prefix + d->T) * (int64_t)d->d) return TSW_EINVAL;
    // Rows per kv head (T * G) bound the kernels' register tiles.
    const int64_t M = (int64_t)d->T * (d->Hq / d->Hkv);
    if (M > 4096) return TSW_EUNSUPPORTED;
    if (d->impl == TSW_IMPL_MFMA) {
        tsw::MfmaConfig cfg;
        if (d->dtype != TSW_DTYPE_BF16 || d->d != 128 || !tsw::mfma_config_for((int)M, &cfg))
            return TSW_EUNSUPPORTED;
    }
    return TSW_OK;
}

// Prefix lists shorter than this go to the vector-ALU kernel under
// TSW_IMPL_AUTO: the work is a few tiles, and its fp32 softmax weights avoid
// the bf16 rounding of P that the matrix path applies, which matters most
// when only a handful of keys carry the weight.
constexpr int64_t kMfmaMinKeys = 256;

bool use_mfma(const tsw_attn_desc* d, int64_t n_keys, tsw::MfmaConfig* cfg) {
    if (d->impl == TSW_IMPL_VALU) return false;
    if (d->dtype != TSW_DTYPE_BF16 || d->d != 128) return false;
    if (d->impl == TSW_IMPL_AUTO && n_keys < kMfmaMinKeys) return false;
    return tsw::mfma_config_for(d->T * (d->Hq / d->Hkv), cfg);
}

// Compute units of the current device, cached per device ordinal.
int device_cus(int* cus) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TSW_EHIP;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return TSW_OK;
        }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return TSW_EHIP;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return TSW_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tiles of the longest slice when n_keys prefix keys are cut into ns parts
// of run_split's chunk size and the last part also takes the tree's tiles.
int64_t longest_slice_tiles(int64_t n_keys, int64_t ns, int64_t tk, int64_t tree_tiles) {
    const int64_t chunk = cdiv(cdiv(n_keys, ns), tk) * tk;
    int64_t last = n_keys - (ns - 1) * chunk;
    if (last < 0) last = 0;
    const int64_t c = chunk / tk, l = cdiv(last, tk) + tree_tiles;
    return c > l ? c : l;
}

// Split-K degree: enough work-groups to occupy every CU once (the matrix
// kernel runs one work-group per CU), no split shorter than two key tiles,
// and gather slices that fit the LDS index buffer.  When a CU is still free
// per kv head and one more split shortens the longest slice (the last one
// carries the tree's own tiles after its share of the prefix), take it: the
// tree rows then get a split of their own or a shorter prefix share.
int plan(const tsw_attn_desc* d, int64_t n_keys, bool gather, int cus, int32_t* n_splits) {
    tsw::MfmaConfig cfg;
    int64_t s;
    if (use_mfma(d, n_keys, &cfg)) {
        const int64_t tk = cfg.tile_keys();
        int64_t smax = cus / d->Hkv;
        if (smax < 1) smax = 1;
        s = smax;
        const int64_t by_len = cdiv(n_keys, 2 * tk);
        if (s > by_len) s = by_len;
        // Every split writes M partial rows of d floats that the merge reads
        // back; below about 3M keys per split that traffic outweighs the
        // split's own K/V bytes (short caches), so take fewer, longer splits.
        const int64_t by_out = n_keys / (3 * (int64_t)d->T * (d->Hq / d->Hkv));
        if (s > by_out) s = by_out;
        if (s < 1) s = 1;
        const int64_t tt = cdiv(d->T, tk);
        if (n_keys > 0 && s + 1 <= smax &&
            longest_slice_tiles(n_keys, s + 1, tk, tt) < longest_slice_tiles(n_keys, s, tk, tt))
            s += 1;
    } else {
        const int64_t nrb = cdiv((int64_t)d->T * (d->Hq / d->Hkv), tsw::kValuRows);
        s = (2 * (int64_t)cus) / (d->Hkv * nrb);
        if (s < 1) s = 1;
        const int64_t by_len = cdiv(n_keys, 2 * tsw::kValuTile);
        if (s > by_len) s = by_len;
    }
    if (gather) {
        const int64_t need = cdiv(n_keys, tsw::kGatherChunkMax);
        if (s < need) s = need;
    } else {
        // (room for the rounding of a part up to whole key tiles)
        const int64_t need = cdiv(n_keys, tsw::kContigChunkMax - 256);
        if (s < need) s = need;
    }
    if (s < 1) s = 1;
    if (s > 65535) return TSW_EUNSUPPORTED;
    *n_splits = (int32_t)s;
    return TSW_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ws_bytes_for(const tsw_attn_desc* d, int32_t n_splits) {
    const size_t rows = (size_t)d->T * d->Hq;
    return align256((size_t)n_splits * rows * d->d * sizeof(float)) +
           align256((size_t)n_splits * rows * sizeof(float));
}

int hip_status(hipError_t e) { return e == hipSuccess ? TSW_OK : TSW_EHIP; }

// root_s (verify only): also write the root row's scores there, one row of
// root_stride floats per query head (matrix-core kernel only).
int run_split(const tsw_attn_desc* d, const void* q, const void* k, const void* v,
              const int32_t* parent, const int32_t* idx, int64_t n_idx, int32_t n_splits,
              float* part_o, float* part_lse, hipStream_t stream, float* root_s = nullptr,
              int64_t root_stride = 0, uint32_t* root_clear = nullptr) {
    const bool gather = idx != nullptr;
    const int64_t n_keys = gather ? n_idx : d->n_prefix;
    SplitArgs a;
    memset(&a, 0, sizeof a);
    int rc = build_mask(parent, d->T, a.mask, nullptr);
    if (rc != TSW_OK) return rc;
    a.q = q;
    a.k = k;
    a.v = v;
    a.idx = idx;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.n_prefix = d->n_prefix;
    a.kv_head_stride = d->kv_head_stride;
    a.n_keys = n_keys;
    a.T = d->T;
    a.Hq = d->Hq;
    a.Hkv = d->Hkv;
    a.G = d->Hq / d->Hkv;
    a.M = a.T * a.G;
    a.n_splits = n_splits;
    a.scale_log2 = d->scale * kLog2e;
    a.B = 1;
    a.root_s = root_s;
    a.root_stride = root_stride;
    a.root_clear = root_clear;

    tsw::MfmaConfig cfg;
    if (use_mfma(d, n_keys, &cfg)) {
        const int64_t tk = cfg.tile_keys();
        a.chunk_keys = cdiv(cdiv(n_keys, n_splits), tk) * tk;
        if (gather && a.chunk_keys > tsw::kGatherChunkMax) return TSW_EUNSUPPORTED;
        if (!gather && a.chunk_keys > tsw::kContigChunkMax) return TSW_EUNSUPPORTED;
        if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15) return TSW_EINVAL;
        if (d->kv_head_stride % 8) return TSW_EINVAL;
        const int mode = gather ? tsw::kModeGather : (root_s ? tsw::kModeContigRoot : tsw::kModeContig);
        return hip_status(tsw::launch_split_mfma(cfg, mode, a, d->Hkv, stream));
    }
    if (root_s) return TSW_EUNSUPPORTED;
    a.chunk_keys = cdiv(cdiv(n_keys, n_splits), tsw::kValuTile) * tsw::kValuTile;
    return hip_status(tsw::launch_split_valu(d->dtype, d->d, gather, a, d->Hkv, stream));
}

int check_common(const tsw_attn_desc* d, const void* q, const void* k, const void* v,
                 const int32_t* parent, const void* o, const void* lse) {
    int rc = check_desc(d);
    if (rc != TSW_OK) return rc;
    if (!q || !k || !v || !parent || !o || !lse) return TSW_EINVAL;
    uint64_t mask[kMaxNodes];
    return build_mask(parent, d->T, mask, nullptr);
}

int full_call(const tsw_attn_desc* d, const void* q, const void* k, const void* v,
              const int32_t* parent, const int32_t* idx, int64_t n_idx, float* o, float* lse,
              void* ws, size_t ws_bytes, tsw_stream_t stream) {
    int rc = check_common(d, q, k, v, parent, o, lse);
    if (rc != TSW_OK) return rc;
    const bool gather = n_idx >= 0;
    if (gather && (n_idx > d->n_prefix)) return TSW_EBADINDEX;
    if (gather && n_idx > 0 && !idx) return TSW_EINVAL;
    if (!ws) return TSW_EINVAL;
    if ((uintptr_t)ws & 255) return TSW_EINVAL;
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != TSW_OK) return rc;
    int32_t n_splits = 0;
    rc = plan(d, gather ? n_idx : d->n_prefix, gather, cus, &n_splits);
    if (rc != TSW_OK) return rc;
    if (ws_bytes < ws_bytes_for(d, n_splits)) return TSW_ENOSPACE;
    const size_t rows = (size_t)d->T * d->Hq;
    float* part_o = (float*)ws;
    float* part_lse = (float*)((char*)ws + align256((size_t)n_splits * rows * d->d * sizeof(float)));
    // An empty index list still needs a non-null pointer for the gather
    // kernel's "partial" mode; no entry of it is read.
    const int32_t* idx_arg = gather ? (idx ? idx : (const int32_t*)ws) : nullptr;
    rc = run_split(d, q, k, v, parent, idx_arg, gather ? n_idx : 0, n_splits, part_o, part_lse,
                   (hipStream_t)stream);
    if (rc != TSW_OK) return rc;
    return hip_status(tsw::launch_lse_merge(n_splits, (int64_t)rows, d->d, part_o, part_lse, o, lse,
                                            (hipStream_t)stream));
}

// Logit slices for the acceptance argmax: about four work-groups per CU
// over all nodes, each slice a multiple of 2048 elements (whole 16-byte
// vectors for every lane of a 256-thread work-group).
constexpr int64_t kAcceptSliceQuantum = 2048;

int accept_plan(int32_t T, int64_t vocab, int64_t* chunk, int32_t* n_chunks) {
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc != TSW_OK) return rc;
    const int64_t per_node = cdiv(4 * (int64_t)cus, T);
    *chunk = cdiv(cdiv(vocab, per_node), kAcceptSliceQuantum) * kAcceptSliceQuantum;
    if (*chunk > tsw::kAcceptSliceMax) *chunk = tsw::kAcceptSliceMax;
    *n_chunks = (int32_t)cdiv(vocab, *chunk);
    return TSW_OK;
}

int check_accept_shape(int32_t T, int64_t vocab) {
    if (T < 1 || T > kMaxNodes) return TSW_EINVAL;
    if (vocab < 1 || vocab > INT32_MAX) return TSW_EINVAL;
    return TSW_OK;
}

// Paged batch: per-split page-table slices live in the 4096-entry LDS
// buffer the gather variant uses for index slices (a few entries are kept
// for the tree rows' pages).
constexpr int64_t kPagedSlicePages = 4080;

int check_paged(const tsw_paged_desc* d, const int64_t* n_prefix, int64_t* n_max, tsw::MfmaConfig* cfg) {
    if (!d || !n_prefix) return TSW_EINVAL;
    if (d->reserved != 0) return TSW_EINVAL;
    if (d->B < 1 || d->B > 64 || d->T < 1 || d->T > kMaxNodes) return TSW_EINVAL;
    if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv != 0) return TSW_EINVAL;
    if (!(d->scale > 0.0f) || !isfinite(d->scale)) return TSW_EINVAL;
    if (d->d != 128 || d->dtype != TSW_DTYPE_BF16) return TSW_EUNSUPPORTED;
    if (d->page_rows < 16 || d->page_rows > 4096 || (d->page_rows & (d->page_rows - 1))) return TSW_EINVAL;
    if (!tsw::mfma_config_for(d->T * (d->Hq / d->Hkv), cfg)) return TSW_EUNSUPPORTED;
    *n_max = 0;
    for (int b = 0; b < d->B; ++b) {
        if (n_prefix[b] < 0) return TSW_EINVAL;
        if (cdiv(n_prefix[b] + d->T, d->page_rows) > d->max_pages) return TSW_EINVAL;
        if (n_prefix[b] > *n_max) *n_max = n_prefix[b];
    }
    return TSW_OK;
}

// Split plan of a batch: about one work-group per CU and kv head for the
// whole batch, dealt so that the longest per-split slice (in key tiles) is as
// short as possible; sequence b gets seg_base[b+1] - seg_base[b] splits (at
// least one) of ceil(len[b] / splits) keys rounded up to whole tiles, and no
// slice longer than max_tiles tiles (what the kernel stages in LDS).  len is
// the committed length (verify) or the index-list length (draft pass).
int plan_segments(const tsw_paged_desc* d, const int64_t* len, const tsw::MfmaConfig& cfg, int64_t max_tiles,
                  int32_t* seg_base) {
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc != TSW_OK) return rc;
    const int64_t tk = cfg.tile_keys();
    int64_t target = cus / d->Hkv;
    if (target < d->B) target = d->B;
    // splits sequence b needs so that none of its slices exceeds `tiles`
    auto splits_for = [&](int64_t b, int64_t tiles) {
        const int64_t nt = cdiv(len[b], tk);
        const int64_t sb = cdiv(nt, tiles);
        return sb < 1 ? (int64_t)1 : sb;
    };
    auto total_for = [&](int64_t tiles) {
        int64_t n = 0;
        for (int b = 0; b < d->B; ++b) n += splits_for(b, tiles);
        return n;
    };
    // smallest per-split tile count whose split total fits the target
    int64_t lo = 2, hi = 2;
    for (int b = 0; b < d->B; ++b) hi = cdiv(len[b], tk) > hi ? cdiv(len[b], tk) : hi;
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (total_for(mid) <= target) hi = mid;
        else lo = mid + 1;
    }
    if (lo > max_tiles) lo = max_tiles;
    seg_base[0] = 0;
    for (int b = 0; b < d->B; ++b) {
        const int64_t sb = splits_for(b, lo);
        if (seg_base[b] + sb > 65535) return TSW_EUNSUPPORTED;
        seg_base[b + 1] = (int32_t)(seg_base[b] + sb);
    }
    return TSW_OK;
}

// Verify: a split's pages must fit the LDS page table.
int plan_paged(const tsw_paged_desc* d, const int64_t* n_prefix, const tsw::MfmaConfig& cfg, int32_t* seg_base) {
    return plan_segments(d, n_prefix, cfg, kPagedSlicePages * d->page_rows / cfg.tile_keys(), seg_base);
}

// Draft pass: a split's index slice must fit the LDS index buffer.
int plan_paged_partial(const tsw_paged_desc* d, const int64_t* n_idx, const tsw::MfmaConfig& cfg,
                       int32_t* seg_base) {
    return plan_segments(d, n_idx, cfg, tsw::kGatherChunkMax / cfg.tile_keys(), seg_base);
}

// Index lists of a paged draft pass: 0 <= n_idx[b] <= n_prefix[b], each
// list within its row of idx_stride entries.
int check_paged_idx(const tsw_paged_desc* d, const int64_t* n_prefix, const int32_t* idx, int64_t idx_stride,
                    const int64_t* n_idx) {
    if (!n_idx) return TSW_EINVAL;
    int64_t most = 0;
    for (int b = 0; b < d->B; ++b) {
        if (n_idx[b] < 0 || n_idx[b] > n_prefix[b]) return TSW_EBADINDEX;
        if (n_idx[b] > most) most = n_idx[b];
    }
    if (most > 0 && !idx) return TSW_EINVAL;
    if (idx_stride < most) return TSW_EINVAL;
    if (most > INT32_MAX) return TSW_EUNSUPPORTED;
    return TSW_OK;
}

// Partials of a paged call: every split holds its own sequence's T x Hq rows.
// Checks shared by the selection entry points (after check_desc).
int check_select(const tsw_attn_desc* d, const void* k, int64_t n_keep, int64_t n_idx, const int32_t* idx) {
    if (d->Hq > tsw::kSelectMaxHeads) return TSW_EUNSUPPORTED;
    if (d->n_prefix > INT32_MAX) return TSW_EUNSUPPORTED;
    if (n_keep < 0 || n_idx < 0) return TSW_EBADINDEX;
    if (!k) return TSW_EINVAL;
    const int64_t n_out = n_idx < d->n_prefix ? n_idx : d->n_prefix;
    if (n_out > 0 && !idx) return TSW_EINVAL;
    const int esz = d->dtype == TSW_DTYPE_F32 ? 4 : 2;
    if ((uintptr_t)k & 15) return TSW_EINVAL;
    if ((d->kv_head_stride * esz) % 16) return TSW_EINVAL;
    return TSW_OK;
}

size_t select_ws_bytes(int64_t n_prefix) {
    const size_t b = align256((size_t)n_prefix * sizeof(float)) + align256(tsw::select_scratch_bytes(n_prefix));
    return b < 256 ? 256 : b;
}

// Verification with selection: the split partials, the root-row scores
// (matrix-core path: Hq rows of root_stride floats), then the selection's
// own workspace.
struct VsLayout {
    int32_t n_splits;
    bool root;
    int64_t root_stride;
    size_t off_root, off_sel, total;
};

int vs_layout(const tsw_attn_desc* d, VsLayout* L) {
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc != TSW_OK) return rc;
    rc = plan(d, d->n_prefix, false, cus, &L->n_splits);
    if (rc != TSW_OK) return rc;
    tsw::MfmaConfig cfg;
    // the kernel writes root scores for head groups of up to 16 (block 0);
    // the 17-24-block shape has no root-score variant (it would spill), so
    // its selection reads K again
    L->root = use_mfma(d, d->n_prefix, &cfg) && d->Hq / d->Hkv <= 16 && !(cfg.rgroups == 8 && cfg.nb >= 3);
    L->root_stride = (d->n_prefix + 3) & ~(int64_t)3;
    L->off_root = ws_bytes_for(d, L->n_splits);
    const size_t root_bytes = L->root ? align256((size_t)d->Hq * L->root_stride * sizeof(float)) : 0;
    L->off_sel = L->off_root + root_bytes;
    L->total = L->off_sel + select_ws_bytes(d->n_prefix);
    return TSW_OK;
}

size_t ws_bytes_paged(const tsw_paged_desc* d, int32_t total_splits) {
    const size_t rows = (size_t)d->T * d->Hq;
    return align256((size_t)total_splits * rows * d->d * sizeof(float)) +
           align256((size_t)total_splits * rows * sizeof(float));
}

}  // namespace

extern "C" {

int tsw_tree_mask_build(const int32_t* parent, int32_t T, uint64_t* mask, int32_t* depth) {
    return build_mask(parent, T, mask, depth);
}

int tsw_plan_splits(const tsw_attn_desc* desc, int64_t n_idx, int32_t* n_splits) {
    int rc = check_desc(desc);
    if (rc != TSW_OK) return rc;
    if (!n_splits) return TSW_EINVAL;
    if (n_idx > desc->n_prefix) return TSW_EBADINDEX;
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != TSW_OK) return rc;
    const bool gather = n_idx >= 0;
    return plan(desc, gather ? n_idx : desc->n_prefix, gather, cus, n_splits);
}

int tsw_workspace_size(const tsw_attn_desc* desc, int64_t n_idx, size_t* bytes) {
    if (!bytes) return TSW_EINVAL;
    int32_t s = 0;
    int rc = tsw_plan_splits(desc, n_idx, &s);
    if (rc != TSW_OK) return rc;
    *bytes = ws_bytes_for(desc, s);
    return TSW_OK;
}

int tsw_tree_attn_verify(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                         const int32_t* parent, float* o, float* lse, void* workspace,
                         size_t workspace_bytes, tsw_stream_t stream) {
    return full_call(desc, q, k, v, parent, nullptr, -1, o, lse, workspace, workspace_bytes, stream);
}

int tsw_tree_attn_partial(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                          const int32_t* parent, const int32_t* idx, int64_t n_idx, float* o,
                          float* lse, void* workspace, size_t workspace_bytes,
                          tsw_stream_t stream) {
    if (n_idx < 0) return TSW_EBADINDEX;
    return full_call(desc, q, k, v, parent, idx, n_idx, o, lse, workspace, workspace_bytes, stream);
}

int tsw_tree_attn_split(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                        const int32_t* parent, const int32_t* idx, int64_t n_idx,
                        int32_t n_splits, float* part_o, float* part_lse, tsw_stream_t stream) {
    int rc = check_common(desc, q, k, v, parent, part_o, part_lse);
    if (rc != TSW_OK) return rc;
    if (n_splits < 1 || n_splits > 65535) return TSW_EINVAL;
    if (idx) {
        if (n_idx < 0 || n_idx > desc->n_prefix) return TSW_EBADINDEX;
    }
    return run_split(desc, q, k, v, parent, idx, idx ? n_idx : 0, n_splits, part_o, part_lse,
                     (hipStream_t)stream);
}

int tsw_lse_merge(int32_t n_splits, int64_t n_rows, int32_t d, const float* part_o,
                  const float* part_lse, float* o, float* lse, tsw_stream_t stream) {
    if (n_splits < 1 || n_rows < 0 || d < 1) return TSW_EINVAL;
    if (n_rows > 0 && (!part_o || !part_lse || !o || !lse)) return TSW_EINVAL;
    return hip_status(tsw::launch_lse_merge(n_splits, n_rows, d, part_o, part_lse, o, lse,
                                            (hipStream_t)stream));
}

int tsw_accept_workspace_size(int32_t T, int64_t vocab, size_t* bytes) {
    if (!bytes) return TSW_EINVAL;
    int rc = check_accept_shape(T, vocab);
    if (rc != TSW_OK) return rc;
    int64_t chunk = 0;
    int32_t n_chunks = 0;
    rc = accept_plan(T, vocab, &chunk, &n_chunks);
    if (rc != TSW_OK) return rc;
    *bytes = align256((size_t)T * n_chunks * sizeof(tsw::AcceptPartial));
    return TSW_OK;
}

namespace {

int accept_call(const int32_t* parent, int32_t T, const void* logits, int64_t vocab, int32_t logits_dtype,
                const int32_t* draft, const int32_t* recent, int64_t n_recent, int32_t window, float theta,
                int32_t* result, void* workspace, size_t workspace_bytes, tsw_stream_t stream) {
    int rc = check_accept_shape(T, vocab);
    if (rc != TSW_OK) return rc;
    tsw::AcceptArgs a;
    memset(&a, 0, sizeof a);
    rc = build_mask(parent, T, a.mask, a.depth);
    if (rc != TSW_OK) return rc;
    if (logits_dtype != TSW_DTYPE_F32 && logits_dtype != TSW_DTYPE_BF16) return TSW_EUNSUPPORTED;
    if (!logits || !draft || !result || !workspace) return TSW_EINVAL;
    if ((uintptr_t)workspace & 7) return TSW_EINVAL;
    int64_t chunk = 0;
    rc = accept_plan(T, vocab, &chunk, &a.n_chunks);
    if (rc != TSW_OK) return rc;
    if (workspace_bytes < (size_t)T * a.n_chunks * sizeof(tsw::AcceptPartial)) return TSW_ENOSPACE;
    a.T = T;
    for (int i = 0; i < T; ++i) a.parent[i] = parent[i];
    a.window = window;
    a.theta = theta;
    a.n_recent = n_recent;
    a.recent = recent;
    const int64_t esz = logits_dtype == TSW_DTYPE_F32 ? 4 : 2;
    const bool vec_ok = ((uintptr_t)logits & 15) == 0 && (vocab * esz) % 16 == 0;
    return hip_status(tsw::launch_accept(a, logits, logits_dtype == TSW_DTYPE_F32 ? 0 : 1, vocab, chunk, vec_ok,
                                         draft, result, (tsw::AcceptPartial*)workspace, (hipStream_t)stream));
}

}  // namespace

int tsw_accept_greedy(const int32_t* parent, int32_t T, const void* logits, int64_t vocab, int32_t logits_dtype,
                      const int32_t* draft, int32_t* result, void* workspace, size_t workspace_bytes,
                      tsw_stream_t stream) {
    return accept_call(parent, T, logits, vocab, logits_dtype, draft, nullptr, 0, 0, 1.0f, result, workspace,
                       workspace_bytes, stream);
}

int tsw_accept_greedy_penalized(const int32_t* parent, int32_t T, const void* logits, int64_t vocab,
                                int32_t logits_dtype, const int32_t* draft, const int32_t* recent, int64_t n_recent,
                                int32_t window, float theta, int32_t* result, void* workspace,
                                size_t workspace_bytes, tsw_stream_t stream) {
    if (window < 0 || window > tsw::kPenaltyMaxWindow || n_recent < 0) return TSW_EINVAL;
    if (!(theta >= 1.0f) || !isfinite(theta)) return TSW_EINVAL;
    if (n_recent > 0 && !recent) return TSW_EINVAL;
    if (theta == 1.0f) window = 0;                    // no penalty: the plain argmax
    return accept_call(parent, T, logits, vocab, logits_dtype, draft, recent, n_recent, window, theta, result,
                       workspace, workspace_bytes, stream);
}

int tsw_context_penalty(const int32_t* parent, int32_t T, void* logits, int64_t vocab, int32_t logits_dtype,
                        const int32_t* draft, const int32_t* recent, int64_t n_recent, int32_t window, float theta,
                        tsw_stream_t stream) {
    int rc = check_accept_shape(T, vocab);
    if (rc != TSW_OK) return rc;
    tsw::PenaltyArgs a;
    memset(&a, 0, sizeof a);
    uint64_t mask[kMaxNodes];
    rc = build_mask(parent, T, mask, nullptr);
    if (rc != TSW_OK) return rc;
    if (logits_dtype != TSW_DTYPE_F32 && logits_dtype != TSW_DTYPE_BF16) return TSW_EUNSUPPORTED;
    if (window < 0 || window > tsw::kPenaltyMaxWindow || n_recent < 0) return TSW_EINVAL;
    if (!(theta >= 1.0f) || !isfinite(theta)) return TSW_EINVAL;
    if (!logits || (T > 1 && !draft) || (n_recent > 0 && !recent)) return TSW_EINVAL;
    if (window == 0 || theta == 1.0f) return TSW_OK;     // nothing changes
    a.T = T;
    a.window = window;
    a.vocab = vocab;
    a.n_recent = n_recent;
    a.theta = theta;
    for (int i = 0; i < T; ++i) a.parent[i] = parent[i];
    return hip_status(tsw::launch_context_penalty(a, logits, logits_dtype == TSW_DTYPE_F32 ? 0 : 1, draft, recent,
                                                  (hipStream_t)stream));
}

int tsw_kv_compact(void* k, void* v, int32_t n_layers, int64_t layer_stride, int32_t Hkv, int32_t d, int32_t dtype,
                   int64_t kv_head_stride, int64_t n_prefix, int32_t T, const int32_t* result,
                   tsw_stream_t stream) {
    if (!k || !v || !result) return TSW_EINVAL;
    if (T < 1 || T > kMaxNodes || n_layers < 1 || n_layers > 65535 || Hkv < 1 || Hkv > 65535) return TSW_EINVAL;
    if (d != 64 && d != 128) return TSW_EUNSUPPORTED;
    if (dtype != TSW_DTYPE_F32 && dtype != TSW_DTYPE_BF16) return TSW_EUNSUPPORTED;
    if (n_prefix < 0) return TSW_EINVAL;
    if (kv_head_stride < (n_prefix + T) * d) return TSW_EINVAL;
    if (n_layers > 1 && layer_stride < (int64_t)Hkv * kv_head_stride) return TSW_EINVAL;
    const int esz = dtype == TSW_DTYPE_F32 ? 4 : 2;
    if (((uintptr_t)k | (uintptr_t)v) & 15) return TSW_EINVAL;
    if ((kv_head_stride * esz) % 16 || (layer_stride * esz) % 16) return TSW_EINVAL;
    tsw::CompactArgs a;
    memset(&a, 0, sizeof a);
    a.k = k;
    a.v = v;
    a.layer_stride = n_layers > 1 ? layer_stride : 0;
    a.kv_head_stride = kv_head_stride;
    a.n_prefix = n_prefix;
    a.T = T;
    a.esz = esz;
    a.row_bytes = d * esz;
    return hip_status(tsw::launch_kv_compact(a, n_layers, Hkv, result, (hipStream_t)stream));
}

int tsw_paged_workspace_size(const tsw_paged_desc* desc, const int64_t* n_prefix, size_t* bytes) {
    if (!bytes) return TSW_EINVAL;
    int64_t n_max = 0;
    tsw::MfmaConfig cfg;
    int rc = check_paged(desc, n_prefix, &n_max, &cfg);
    if (rc != TSW_OK) return rc;
    int32_t seg_base[65];
    rc = plan_paged(desc, n_prefix, cfg, seg_base);
    if (rc != TSW_OK) return rc;
    *bytes = ws_bytes_paged(desc, seg_base[desc->B]);
    return TSW_OK;
}

int tsw_paged_partial_workspace_size(const tsw_paged_desc* desc, const int64_t* n_prefix, const int64_t* n_idx,
                                     size_t* bytes) {
    if (!bytes) return TSW_EINVAL;
    int64_t n_max = 0;
    tsw::MfmaConfig cfg;
    int rc = check_paged(desc, n_prefix, &n_max, &cfg);
    if (rc != TSW_OK) return rc;
    if (!n_idx) return TSW_EINVAL;
    for (int b = 0; b < desc->B; ++b)
        if (n_idx[b] < 0 || n_idx[b] > n_prefix[b]) return TSW_EBADINDEX;
    int32_t seg_base[65];
    rc = plan_paged_partial(desc, n_idx, cfg, seg_base);
    if (rc != TSW_OK) return rc;
    *bytes = ws_bytes_paged(desc, seg_base[desc->B]);
    return TSW_OK;
}

namespace {

// Both paged calls: the split over every sequence's key list (its committed
// positions, or its index list when idx_list is set), then the merge of each
// sequence's parts.
int paged_call(const tsw_paged_desc* desc, const void* q, const void* k_pages, const void* v_pages,
               const int32_t* block_table, const int64_t* n_prefix, const int32_t* parent, const int32_t* idx_list,
               int64_t idx_stride, const int64_t* n_idx, float* o, float* lse, void* workspace,
               size_t workspace_bytes, tsw_stream_t stream) {
    int64_t n_max = 0;
    tsw::MfmaConfig cfg;
    int rc = check_paged(desc, n_prefix, &n_max, &cfg);
    if (rc != TSW_OK) return rc;
    const bool gather = n_idx != nullptr;
    if (gather) {
        rc = check_paged_idx(desc, n_prefix, idx_list, idx_stride, n_idx);
        if (rc != TSW_OK) return rc;
    }
    if (!q || !k_pages || !v_pages || !block_table || !parent || !o || !lse || !workspace) return TSW_EINVAL;
    if (((uintptr_t)q | (uintptr_t)k_pages | (uintptr_t)v_pages) & 15) return TSW_EINVAL;
    if ((uintptr_t)workspace & 255) return TSW_EINVAL;
    SplitArgs a;
    memset(&a, 0, sizeof a);
    rc = build_mask(parent, desc->T, a.mask, nullptr);
    if (rc != TSW_OK) return rc;
    rc = gather ? plan_paged_partial(desc, n_idx, cfg, a.seg_base) : plan_paged(desc, n_prefix, cfg, a.seg_base);
    if (rc != TSW_OK) return rc;
    const int32_t n_splits = a.seg_base[desc->B];
    if (workspace_bytes < ws_bytes_paged(desc, n_splits)) return TSW_ENOSPACE;
    const size_t rows_per_seq = (size_t)desc->T * desc->Hq;
    float* part_o = (float*)workspace;
    float* part_lse =
        (float*)((char*)workspace + align256((size_t)n_splits * rows_per_seq * desc->d * sizeof(float)));
    a.q = q;
    a.k = k_pages;
    a.v = v_pages;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.T = desc->T;
    a.Hq = desc->Hq;
    a.Hkv = desc->Hkv;
    a.G = desc->Hq / desc->Hkv;
    a.M = a.T * a.G;
    a.n_splits = n_splits;
    a.scale_log2 = desc->scale * kLog2e;
    a.B = desc->B;
    a.table = block_table;
    a.table_stride = desc->max_pages;
    a.page_rows = desc->page_rows;
    int shift = 0;
    while ((1 << shift) < desc->page_rows) ++shift;
    a.page_shift = shift;
    a.page_bytes = (int64_t)desc->Hkv * desc->page_rows * desc->d * 2;
    for (int b = 0; b < desc->B; ++b) a.npb[b] = n_prefix[b];
    if (gather) {
        for (int b = 0; b < desc->B; ++b) a.nib[b] = n_idx[b];
        // an all-empty batch still passes a non-null list; no entry is read
        a.idx = idx_list ? idx_list : (const int32_t*)workspace;
        a.idx_stride = idx_stride;
    }
    rc = hip_status(tsw::launch_split_mfma(cfg, gather ? tsw::kModePagedGather : tsw::kModePaged, a, desc->Hkv,
                                           (hipStream_t)stream));
    if (rc != TSW_OK) return rc;
    tsw::MergeSegs segs;
    memset(&segs, 0, sizeof segs);
    segs.n_seg = desc->B;
    segs.rows_per_seg = (int64_t)rows_per_seq;
    for (int b = 0; b <= desc->B; ++b) segs.base[b] = a.seg_base[b];
    return hip_status(tsw::launch_lse_merge_segs(segs, (int64_t)rows_per_seq * desc->B, part_o, part_lse, o, lse,
                                                 (hipStream_t)stream));
}

}  // namespace

int tsw_tree_attn_verify_paged(const tsw_paged_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int64_t* n_prefix, const int32_t* parent, float* o,
                               float* lse, void* workspace, size_t workspace_bytes, tsw_stream_t stream) {
    return paged_call(desc, q, k_pages, v_pages, block_table, n_prefix, parent, nullptr, 0, nullptr, o, lse,
                      workspace, workspace_bytes, stream);
}

int tsw_tree_attn_partial_paged(const tsw_paged_desc* desc, const void* q, const void* k_pages, const void* v_pages,
                                const int32_t* block_table, const int64_t* n_prefix, const int32_t* parent,
                                const int32_t* idx, int64_t idx_stride, const int64_t* n_idx, float* o, float* lse,
                                void* workspace, size_t workspace_bytes, tsw_stream_t stream) {
    if (!n_idx) return TSW_EINVAL;
    return paged_call(desc, q, k_pages, v_pages, block_table, n_prefix, parent, idx, idx_stride, n_idx, o, lse,
                      workspace, workspace_bytes, stream);
}

int tsw_select_workspace_size(int64_t n_prefix, size_t* bytes) {
    if (!bytes || n_prefix < 0 || n_prefix > INT32_MAX) return TSW_EINVAL;
    *bytes = select_ws_bytes(n_prefix);
    return TSW_OK;
}

int tsw_select_partial(const tsw_attn_desc* desc, const void* q, const void* k, const float* lse, int64_t n_keep,
                       int64_t n_idx, int32_t* idx, float* importance, void* workspace, size_t workspace_bytes,
                       tsw_stream_t stream) {
    int rc = check_desc(desc);
    if (rc != TSW_OK) return rc;
    rc = check_select(desc, k, n_keep, n_idx, idx);
    if (rc != TSW_OK) return rc;
    if (!q || !lse) return TSW_EINVAL;
    const int64_t n_out = n_idx < desc->n_prefix ? n_idx : desc->n_prefix;
    if (!workspace) return TSW_EINVAL;
    if ((uintptr_t)workspace & 255) return TSW_EINVAL;
    const size_t imp_bytes = align256((size_t)desc->n_prefix * sizeof(float));
    if (workspace_bytes < imp_bytes + tsw::select_scratch_bytes(desc->n_prefix)) return TSW_ENOSPACE;
    float* imp = importance ? importance : (float*)workspace;
    uint32_t* scratch = (uint32_t*)((char*)workspace + imp_bytes);
    tsw::SelectArgs a;
    memset(&a, 0, sizeof a);
    a.q = q;
    a.k = k;
    a.lse = lse;
    a.n_prefix = desc->n_prefix;
    a.kv_head_stride = desc->kv_head_stride;
    a.Hq = desc->Hq;
    a.Hkv = desc->Hkv;
    a.G = desc->Hq / desc->Hkv;
    a.d = desc->d;
    a.dtype = desc->dtype == TSW_DTYPE_F32 ? 0 : 1;
    a.scale = desc->scale;
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != TSW_OK) return rc;
    rc = hip_status(tsw::launch_importance(a, imp, cus, (hipStream_t)stream));
    if (rc != TSW_OK || n_out == 0) return rc;
    const int64_t keep = n_keep < n_out ? n_keep : n_out;
    return hip_status(tsw::launch_select(imp, desc->n_prefix, keep, n_out, idx, scratch, (hipStream_t)stream));
}

int tsw_verify_select_workspace_size(const tsw_attn_desc* desc, size_t* bytes) {
    if (!bytes) return TSW_EINVAL;
    int rc = check_desc(desc);
    if (rc != TSW_OK) return rc;
    if (desc->n_prefix > INT32_MAX) return TSW_EUNSUPPORTED;
    VsLayout L;
    rc = vs_layout(desc, &L);
    if (rc != TSW_OK) return rc;
    *bytes = L.total;
    return TSW_OK;
}

int tsw_tree_attn_verify_select(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                                const int32_t* parent, float* o, float* lse, int64_t n_keep, int64_t n_idx,
                                int32_t* idx, float* importance, void* workspace, size_t workspace_bytes,
                                tsw_stream_t stream) {
    int rc = check_common(desc, q, k, v, parent, o, lse);
    if (rc != TSW_OK) return rc;
    rc = check_select(desc, k, n_keep, n_idx, idx);
    if (rc != TSW_OK) return rc;
    if (!workspace || ((uintptr_t)workspace & 255)) return TSW_EINVAL;
    VsLayout L;
    rc = vs_layout(desc, &L);
    if (rc != TSW_OK) return rc;
    if (workspace_bytes < L.total) return TSW_ENOSPACE;
    const size_t rows = (size_t)desc->T * desc->Hq;
    char* ws = (char*)workspace;
    float* part_o = (float*)ws;
    float* part_lse = (float*)(ws + align256((size_t)L.n_splits * rows * desc->d * sizeof(float)));
    float* root_s = L.root ? (float*)(ws + L.off_root) : nullptr;
    char* sel = ws + L.off_sel;
    float* imp = importance ? importance : (float*)sel;
    uint32_t* scratch = (uint32_t*)(sel + align256((size_t)desc->n_prefix * sizeof(float)));
    hipStream_t st = (hipStream_t)stream;

    // the split kernel zeroes the selection's digit totals (scratch[0..1024))
    rc = run_split(desc, q, k, v, parent, nullptr, 0, L.n_splits, part_o, part_lse, st, root_s, L.root_stride,
                   L.root ? scratch : nullptr);
    if (rc != TSW_OK) return rc;
    rc = hip_status(tsw::launch_lse_merge(L.n_splits, (int64_t)rows, desc->d, part_o, part_lse, o, lse, st));
    if (rc != TSW_OK) return rc;

    const int64_t n_out = n_idx < desc->n_prefix ? n_idx : desc->n_prefix;
    const int64_t keep = n_keep < n_out ? n_keep : n_out;
    if (!L.root) {
        // vector-ALU verification: importance from K as in tsw_select_partial
        tsw::SelectArgs a;
        memset(&a, 0, sizeof a);
        a.q = q;
        a.k = k;
        a.lse = lse;
        a.n_prefix = desc->n_prefix;
        a.kv_head_stride = desc->kv_head_stride;
        a.Hq = desc->Hq;
        a.Hkv = desc->Hkv;
        a.G = desc->Hq / desc->Hkv;
        a.d = desc->d;
        a.dtype = desc->dtype == TSW_DTYPE_F32 ? 0 : 1;
        a.scale = desc->scale;
        int cus = 0;
        rc = device_cus(&cus);
        if (rc != TSW_OK) return rc;
        rc = hip_status(tsw::launch_importance(a, imp, cus, st));
        if (rc != TSW_OK || n_out == 0) return rc;
        return hip_status(tsw::launch_select(imp, desc->n_prefix, keep, n_out, idx, scratch, st));
    }
    const float c = desc->scale * kLog2e;
    // importance, the kept positions and the first radix pass's counts, then
    // the remaining passes
    rc = hip_status(tsw::launch_importance_from_scores(root_s, L.root_stride, lse, desc->Hq, desc->n_prefix, c,
                                                       keep, imp, n_out > 0 ? scratch : nullptr, idx, st));
    if (rc != TSW_OK || n_out == 0) return rc;
    if (rc != TSW_OK) return rc;
    return hip_status(tsw::launch_select_passes(imp, desc->n_prefix, keep, n_out, idx, scratch, 1, st));
}

int tsw_read_stream(const tsw_attn_desc* desc, const void* k, const void* v, unsigned* sink, tsw_stream_t stream) {
    int rc = check_desc(desc);
    if (rc != TSW_OK) return rc;
    if (!k || !v || !sink) return TSW_EINVAL;
    if (desc->dtype != TSW_DTYPE_BF16 || desc->d != 128) return TSW_EUNSUPPORTED;
    if (((uintptr_t)k | (uintptr_t)v) & 15) return TSW_EINVAL;
    if (desc->kv_head_stride % 8) return TSW_EINVAL;
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != TSW_OK) return rc;
    int32_t n_splits = 0;
    rc = plan(desc, desc->n_prefix, false, cus, &n_splits);
    if (rc != TSW_OK) return rc;
    const int64_t rows = desc->n_prefix + desc->T;
    return hip_status(tsw::launch_read_stream(k, v, desc->Hkv, desc->kv_head_stride * 2, rows, n_splits, sink,
                                              (hipStream_t)stream));
}

int tsw_launch_floor(const tsw_attn_desc* desc, int64_t n_idx, int32_t* threads, tsw_stream_t stream) {
    int rc = check_desc(desc);
    if (rc != TSW_OK) return rc;
    if (n_idx > desc->n_prefix) return TSW_EBADINDEX;
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != TSW_OK) return rc;
    const bool gather = n_idx >= 0;
    const int64_t n_keys = gather ? n_idx : desc->n_prefix;
    SplitArgs a;
    memset(&a, 0, sizeof a);
    rc = plan(desc, n_keys, gather, cus, &a.n_splits);
    if (rc != TSW_OK) return rc;
    tsw::MfmaConfig cfg;
    // the vector-ALU split kernel runs 256 threads per work-group
    const int nthreads = use_mfma(desc, n_keys, &cfg) ? cfg.waves * 64 : 256;
    if (threads) *threads = nthreads;
    return hip_status(tsw::launch_launch_floor(a, desc->Hkv, nthreads, (hipStream_t)stream));
}

const char* tsw_status_str(int status) {
    switch (status) {
        case TSW_OK: return "ok";
        case TSW_EINVAL: return "invalid argument";
        case TSW_EBADTREE: return "parent[] is not a tree rooted at node 0 with parents before children";
        case TSW_EBADINDEX: return "index list size out of range";
        case TSW_EUNSUPPORTED: return "unsupported head dim, dtype, shape or implementation";
        case TSW_ENOSPACE: return "workspace too small";
        case TSW_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

}  // extern "C"
