/*
 * tsw.h -- C ABI of the tree-verification attention library for AMD MI355X
 * (gfx950).
 *
 * The operation.  In TokenSwift's generation loop the drafted candidate
 * tokens form a token tree (a simple 3-ary tree) and are verified in one
 * forward pass with tree-structured attention against the full KV cache;
 * the result must equal what the target model computes for each candidate
 * on its own (lossless).  The draft pass runs the same model over a partial
 * KV cache that always keeps the initial positions and a selection of later
 * ones.  Sources:
 *   - "TokenSwift - A framework for accelerating the generation of ultra-long
 *     text" (aiboss88 project page), technical principles: tree-based
 *     multi-candidate verification; dynamic KV cache update.
 *   - "90分钟生成10万Token，新框架实现3倍无损加速超长文本生成" (Tencent Cloud
 *     article), 技术原理 figure text (verification with the full KV cache,
 *     tree-based attention) and 优势与特点 / 无损的输出质量 (the draft model is
 *     the target model with a partial KV cache).
 *   - "From Hours to Minutes: Lossless Acceleration of Ultra Long Sequence
 *     Generation up to 100K Tokens" (arxivlens summary), Technical
 *     Contribution: 3-ary tree, KV compression.
 *
 * For tree node i (0 <= i < T) and query head h, with kv head g = h / (Hq/Hkv):
 *   visible(i) = prefix  u  { n_prefix + j : j is i or an ancestor of i }
 *   prefix     = {0 .. n_prefix-1}                  (tsw_tree_attn_verify)
 *              = {idx[0] .. idx[n_idx-1]}           (tsw_tree_attn_partial)
 *   s_p        = scale * dot(Q[i][h][:], K[g][p][:])        p in visible(i)
 *   O[i][h][:] = sum_p exp(s_p) V[g][p][:] / sum_p exp(s_p)
 *   LSE[i][h]  = ln(sum_p exp(s_p))
 * The tree's own K/V rows are stored in the cache right after the committed
 * prefix: node j at position n_prefix + j.
 *
 * Memory layout (all row-major, element type per desc->dtype):
 *   q    [T][Hq][d]                       device, contiguous
 *   k, v [Hkv][rows][d]                   device, kv_head_stride elements
 *                                         between heads, rows >= n_prefix + T
 *   o    [T][Hq][d]   float32             device
 *   lse  [T][Hq]      float32             device, natural log
 *   parent [T] int32                      HOST memory; parent[0] = -1 and
 *                                         0 <= parent[i] < i for i >= 1
 *   idx  [n_idx] int32                    device; sorted ascending, distinct,
 *                                         every entry in [0, n_prefix)
 *
 * Ownership and errors.  The caller owns every buffer.  The library never
 * allocates or frees memory and never synchronises: compute calls enqueue
 * kernels on `stream` and return.  Host arguments (desc, parent) are read
 * before the call returns.  Device buffers must stay valid until the stream
 * work completes; o/lse/workspace must not overlap the inputs or each other.
 * All argument checks run before any HIP call; on an error nothing is
 * launched and the outputs are untouched.  idx validity is a precondition
 * (it lives on the device and is not inspected); violating it gives
 * unspecified results but no out-of-bounds access as long as every entry is
 * in [0, n_prefix).  Functions return TSW_OK (0) or a negative status.
 */
#ifndef TSW_H
#define TSW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TSW_OK = 0,
    TSW_EINVAL = -1,       /* null pointer, bad size, stride, scale or reserved field */
    TSW_EBADTREE = -2,     /* parent[] is not a tree rooted at node 0 in topological order */
    TSW_EBADINDEX = -3,    /* n_idx < 0 or n_idx > n_prefix */
    TSW_EUNSUPPORTED = -4, /* head dim, dtype or implementation choice not supported */
    TSW_ENOSPACE = -5,     /* workspace smaller than tsw_workspace_size() */
    TSW_EHIP = -6          /* a HIP runtime call failed (no device, launch failure) */
};

enum { TSW_DTYPE_F32 = 0, TSW_DTYPE_BF16 = 1 };

/* Kernel family choice.  AUTO takes the matrix-core (MFMA) kernel for
 * bfloat16 with d = 128, at most 384 query rows T * (Hq / Hkv) per kv head
 * and at least 256 keys, else the vector-ALU kernel.  MFMA outside its
 * shapes returns TSW_EUNSUPPORTED. */
enum { TSW_IMPL_AUTO = 0, TSW_IMPL_VALU = 1, TSW_IMPL_MFMA = 2 };

/* A cache stream handle: a hipStream_t (NULL = the legacy default stream). */
typedef void* tsw_stream_t;

typedef struct tsw_attn_desc {
    int32_t T;              /* tree nodes (query tokens), 1..64 */
    int32_t Hq;             /* query heads, >= 1 */
    int32_t Hkv;            /* kv heads, >= 1, Hq % Hkv == 0 */
    int32_t d;              /* head dim: 64 or 128 */
    int64_t n_prefix;       /* committed cache positions, >= 0 */
    int64_t kv_head_stride; /* elements between kv heads in k and v, >= (n_prefix + T) * d */
    int32_t dtype;          /* TSW_DTYPE_F32 or TSW_DTYPE_BF16, for q, k and v */
    int32_t impl;           /* TSW_IMPL_* */
    float scale;            /* score scale, positive and finite (1/sqrt(d) usually) */
    int32_t reserved;       /* must be 0 */
} tsw_attn_desc;

/* Builds the tree mask on the host: bit j of mask[i] is set iff node j is
 * node i or an ancestor of i; depth[i] = edges from the root (may be NULL).
 * parent, mask, depth are host arrays of length T, 1 <= T <= 64.
 * Errors: TSW_EINVAL (null pointer, T out of range), TSW_EBADTREE. */
int tsw_tree_mask_build(const int32_t* parent, int32_t T, uint64_t* mask, int32_t* depth);

/* Number of KV splits the library uses for this problem on the current
 * device (the split-K degree of tsw_tree_attn_verify / _partial).  n_idx < 0
 * selects the verify variant.  Needs a HIP device (queries its CU count). */
int tsw_plan_splits(const tsw_attn_desc* desc, int64_t n_idx, int32_t* n_splits);

/* Workspace bytes tsw_tree_attn_verify (n_idx < 0) or tsw_tree_attn_partial
 * (n_idx >= 0) need on the current device: the per-split partial results
 * n_splits * T * Hq * (d + 1) float32 plus alignment. */
int tsw_workspace_size(const tsw_attn_desc* desc, int64_t n_idx, size_t* bytes);

/* Tree verification against the full cache: O and LSE for every (node,
 * query head).  workspace: device memory of at least tsw_workspace_size()
 * bytes, 256-byte aligned, contents need not be initialised. */
int tsw_tree_attn_verify(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                         const int32_t* parent, float* o, float* lse, void* workspace,
                         size_t workspace_bytes, tsw_stream_t stream);

/* Draft-pass variant: the prefix is the index list idx[0..n_idx) (device
 * memory, sorted, distinct, < n_prefix) instead of all committed positions;
 * the tree rows are attended under the tree mask as in verify.  n_idx = 0
 * attends to the tree rows only. */
int tsw_tree_attn_partial(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                          const int32_t* parent, const int32_t* idx, int64_t n_idx, float* o,
                          float* lse, void* workspace, size_t workspace_bytes,
                          tsw_stream_t stream);

/* First phase on its own: split the prefix key list (all positions when
 * idx == NULL, else idx[0..n_idx)) into n_splits contiguous parts and write,
 * for every part s and row (node, head), the attention result over that part
 * normalised within the part, and its LSE:
 *   part_o   [n_splits][T][Hq][d] float32 (device)
 *   part_lse [n_splits][T][Hq]    float32 (device), -inf when the part holds
 *                                 no visible key for the row.
 * The last part also holds the tree rows.  n_splits >= 1; parts may be
 * empty.  Combining the parts with tsw_lse_merge gives the verify / partial
 * result; the same merge combines parts computed on different devices.
 * On the matrix-core path a contiguous part holds at most 2^23 keys (larger
 * parts: TSW_EUNSUPPORTED; tsw_plan_splits plans parts within the limit). */
int tsw_tree_attn_split(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                        const int32_t* parent, const int32_t* idx, int64_t n_idx,
                        int32_t n_splits, float* part_o, float* part_lse, tsw_stream_t stream);

/* Second phase: merge n_splits partial attention results over disjoint key
 * sets into the result over their union:
 *   LSE = ln(sum_s exp(L_s)),  O = sum_s exp(L_s - LSE) O_s
 * part_o [n_splits][n_rows][d], part_lse [n_splits][n_rows] (natural log,
 * -inf for empty parts), o [n_rows][d], lse [n_rows]; all float32 device
 * memory.  Rows whose parts are all empty get O = 0 and LSE = -inf. */
int tsw_lse_merge(int32_t n_splits, int64_t n_rows, int32_t d, const float* part_o,
                  const float* part_lse, float* o, float* lse, tsw_stream_t stream);

/* ---------------------------------------------------------------------
 * Paged batch: B sequences that share one tree shape (same T and parent[])
 * but each have their own committed length n_prefix[b] and their own queries,
 * with K and V stored in fixed-size pages of one pool.  Per sequence the
 * result is exactly tsw_tree_attn_verify's on that sequence's cache.
 *   q      [B][T][Hq][d]                        device
 *   k_pages, v_pages [n_pages][Hkv][page_rows][d]  device page pools
 *   block_table [B][max_pages] int32            device; sequence b's cache
 *          position p lives in page block_table[b*max_pages + p/page_rows],
 *          row p % page_rows; node j of the tree at position n_prefix[b] + j
 *   n_prefix [B] int64                          HOST
 *   o [B][T][Hq][d], lse [B][T][Hq] float32     device
 * Only the matrix-core kernel serves this call (bfloat16, d = 128, at most
 * 384 query rows per kv head): P is rounded to bfloat16 before P V, so with
 * fewer than a few hundred visible keys the error can exceed that of the
 * vector-ALU kernel.  The block-table entries a sequence needs must name
 * pages of the pool (a precondition; they are read on the device).
 * ------------------------------------------------------------------- */
typedef struct tsw_paged_desc {
    int32_t B;              /* sequences, 1..64 */
    int32_t T, Hq, Hkv;     /* as in tsw_attn_desc */
    int32_t d;              /* 128 */
    int32_t page_rows;      /* rows per page: a power of two, 16..4096 */
    int32_t max_pages;      /* entries per block-table row, >= ceil((n_prefix[b]+T)/page_rows) */
    int32_t dtype;          /* TSW_DTYPE_BF16 */
    float scale;            /* positive and finite */
    int32_t reserved;       /* must be 0 */
} tsw_paged_desc;

/* Workspace bytes for a paged call with these lengths on the current device. */
int tsw_paged_workspace_size(const tsw_paged_desc* desc, const int64_t* n_prefix, size_t* bytes);

/* Errors: TSW_EINVAL (shape, lengths, pointers, alignment: q/k/v 16 bytes,
 * workspace 256), TSW_EBADTREE, TSW_EUNSUPPORTED (dtype, d, too many rows
 * per kv head), TSW_ENOSPACE, TSW_EHIP. */
int tsw_tree_attn_verify_paged(const tsw_paged_desc* desc, const void* q, const void* k_pages,
                               const void* v_pages, const int32_t* block_table,
                               const int64_t* n_prefix, const int32_t* parent, float* o, float* lse,
                               void* workspace, size_t workspace_bytes, tsw_stream_t stream);

/* Paged draft pass.  The draft model is the target model reading a partial
 * KV cache ("90分钟生成10万Token…" (Tencent Cloud), 优势与特点 / 无损的输出质量;
 * "TokenSwift - A framework…" (aiboss88), technical principles, dynamic KV
 * cache update); over a batch of sequences in one page pool, each sequence's
 * result is exactly tsw_tree_attn_partial's on that sequence's cache with its
 * own index list:
 *   idx   [B][idx_stride] int32   device; sequence b's list is
 *         idx[b*idx_stride .. b*idx_stride + n_idx[b]), sorted ascending,
 *         distinct, every entry in [0, n_prefix[b]) (a precondition, read on
 *         the device); idx may be NULL when every n_idx[b] is 0
 *   n_idx [B] int64               HOST; 0 <= n_idx[b] <= n_prefix[b]
 *                                 (n_idx[b] = 0: the tree rows only)
 *   idx_stride                    >= max n_idx[b]
 * Tree node j still reads position n_prefix[b] + j through the block table.
 * The pool must hold fewer than 2^32 rows per kv head (pages x page_rows);
 * q, the pools, block_table, parent, o, lse and the workspace are as for
 * tsw_tree_attn_verify_paged.  Errors: as that call, plus TSW_EBADINDEX (an
 * n_idx[b] out of range) and TSW_EINVAL (idx_stride too small, idx NULL with
 * a non-empty list). */
int tsw_paged_partial_workspace_size(const tsw_paged_desc* desc, const int64_t* n_prefix,
                                     const int64_t* n_idx, size_t* bytes);
int tsw_tree_attn_partial_paged(const tsw_paged_desc* desc, const void* q, const void* k_pages,
                                const void* v_pages, const int32_t* block_table,
                                const int64_t* n_prefix, const int32_t* parent, const int32_t* idx,
                                int64_t idx_stride, const int64_t* n_idx, float* o, float* lse,
                                void* workspace, size_t workspace_bytes, tsw_stream_t stream);

/* ---------------------------------------------------------------------
 * Partial-cache selection for the next draft pass.  The draft pass keeps the
 * initial positions and the most important others ("TokenSwift - A framework
 * for accelerating the generation of ultra-long text" (aiboss88), technical
 * principles, dynamic KV cache update).  The pages do not define
 * importance; here it is the attention mass the tree root's query heads put
 * on each committed position in the verification pass:
 *   imp[p] = sum_h exp(scale * q[0][h] . k[g(h)][p] - lse[0][h]),  p < n_prefix
 * (q, k as passed to tsw_tree_attn_verify, lse its output).  The index list
 * is 0 .. n_keep-1 followed by the n_idx - n_keep positions >= n_keep of
 * largest importance (equal importance: the lower position first), sorted
 * ascending: ready for tsw_tree_attn_partial.
 * ------------------------------------------------------------------- */

/* Workspace bytes for n_prefix committed positions (importance values and
 * selection counts). */
int tsw_select_workspace_size(int64_t n_prefix, size_t* bytes);

/* desc as for verification (Hq <= 64, n_prefix < 2^31); k 16-byte aligned.
 * Writes idx[0 .. min(n_idx, n_prefix)) (device int32).  importance:
 * optional device float32 [n_prefix] output of imp (NULL: kept in the
 * workspace).  workspace: device, 256-byte aligned, >=
 * tsw_select_workspace_size() bytes, scratch.  Errors: TSW_EINVAL,
 * TSW_EBADINDEX (negative n_keep or n_idx), TSW_EUNSUPPORTED, TSW_ENOSPACE,
 * TSW_EHIP. */
int tsw_select_partial(const tsw_attn_desc* desc, const void* q, const void* k, const float* lse,
                       int64_t n_keep, int64_t n_idx, int32_t* idx, float* importance, void* workspace,
                       size_t workspace_bytes, tsw_stream_t stream);

/* Verification and selection in one call: tsw_tree_attn_verify's o and lse,
 * then tsw_select_partial's idx and importance for the same desc, q and k.
 * On the matrix-core path the verification kernel writes the root row's
 * scores dot(q[0][h], k[g(h)][p]) (p < n_prefix) to the workspace as it
 * streams K, and the importance is formed from them, so K is read once;
 * otherwise the importance is computed from q and k as in
 * tsw_select_partial.  Selection arguments and errors as for
 * tsw_select_partial, the rest as for tsw_tree_attn_verify; workspace:
 * device, 256-byte aligned, >= tsw_verify_select_workspace_size() bytes. */
int tsw_verify_select_workspace_size(const tsw_attn_desc* desc, size_t* bytes);
int tsw_tree_attn_verify_select(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                                const int32_t* parent, float* o, float* lse, int64_t n_keep, int64_t n_idx,
                                int32_t* idx, float* importance, void* workspace, size_t workspace_bytes,
                                tsw_stream_t stream);

/* ---------------------------------------------------------------------
 * After verification: greedy acceptance and accepted-path KV compaction.
 *
 * The target model's logits at each tree node give its most likely next
 * token there (first index among equal maxima).  Node i > 0 is accepted when
 * its parent is accepted and draft[i] equals that token at parent[i]; the
 * root (node 0, the committed token) is always accepted.  The output path is
 * the root path of the deepest accepted node (lowest index among equally
 * deep ones), and the bonus token is the target's most likely token after
 * it.  Sources: "TokenSwift - A framework for accelerating the generation of
 * ultra-long text" (aiboss88), technical principles, tree-based
 * multi-candidate token verification (the longest valid candidate is kept;
 * the output stays consistent with the target model); Tencent Cloud article
 * "90分钟生成10万Token，新框架实现3倍无损加速超长文本生成", 技术原理
 * (parallel-verification figure text: the longest valid sequence is kept).
 * The pages pick randomly among equally long candidates or just "the
 * longest"; this library takes the lowest node index, which never matters
 * when sibling tokens are distinct.
 * ------------------------------------------------------------------- */

/* Workspace bytes tsw_accept_greedy needs for T nodes and this vocabulary
 * on the current device.  TSW_EINVAL for T outside 1..64 or vocab outside
 * 1..2^31-1. */
int tsw_accept_workspace_size(int32_t T, int64_t vocab, size_t* bytes);

/* logits [T][vocab] (device, float32 or bfloat16 per logits_dtype, rows
 * contiguous), draft [T] int32 (device; draft[0] is not read), parent [T]
 * int32 (HOST, same encoding as above).  Writes result (device, int32,
 * 2 + 2*T entries): result[0] = L (path length, 1..T), result[1] = bonus
 * token, result[2 .. 2+L) = the path's node indices from the root,
 * result[2+L .. 2+T) = -1, result[2+T .. 2+2T) = the most likely token at
 * every node.  workspace: device, >= tsw_accept_workspace_size() bytes,
 * 8-byte aligned, scratch.  NaN logits are outside the contract (a row of
 * NaN reports token 0).  Errors: TSW_EINVAL, TSW_EBADTREE, TSW_EUNSUPPORTED
 * (dtype), TSW_ENOSPACE, TSW_EHIP. */
int tsw_accept_greedy(const int32_t* parent, int32_t T, const void* logits, int64_t vocab,
                      int32_t logits_dtype, const int32_t* draft, int32_t* result, void* workspace,
                      size_t workspace_bytes, tsw_stream_t stream);

/* Contextual penalty on the target logits of every tree node, in place,
 * before tsw_accept_greedy ("TokenSwift - A framework for accelerating the
 * generation of ultra-long text" (aiboss88), technical principles,
 * contextual penalty strategy: recently generated tokens are penalised; the
 * form and window are this library's reading, the usual repetition
 * penalty).  Node t's window is the last `window` tokens of recent[0 ..
 * n_recent) (the committed tokens, oldest first; the last one is the root's)
 * followed by draft[] along the path from the root down to t (depth 1 ..
 * depth(t)): what sequential generation had produced before predicting the
 * token after t.  For every distinct id v in it with 0 <= v < vocab,
 * logits[t][v] becomes l / theta when l > 0, else l * theta (float32
 * arithmetic, correctly rounded; bfloat16 logits are widened and the result
 * rounded to nearest even).  Other ids are ignored.
 *   parent [T] int32   HOST, as for tsw_tree_attn_verify
 *   logits [T][vocab]  device, float32 or bfloat16 (logits_dtype), modified
 *   draft  [T] int32   device (draft[0] unused); recent [n_recent] int32 device
 * window in 0 .. 8192, theta >= 1 and finite; window 0 or theta 1 launch
 * nothing.  Errors: TSW_EINVAL, TSW_EBADTREE, TSW_EUNSUPPORTED, TSW_EHIP. */
int tsw_context_penalty(const int32_t* parent, int32_t T, void* logits, int64_t vocab, int32_t logits_dtype,
                        const int32_t* draft, const int32_t* recent, int64_t n_recent, int32_t window, float theta,
                        tsw_stream_t stream);

/* tsw_accept_greedy on the logits as tsw_context_penalty would leave them,
 * without modifying them: each argmax work-group applies the penalty to the
 * window tokens in its own slice of the vocabulary as it scans, so the step
 * costs about one plain acceptance.  Arguments as for the two calls; the
 * workspace is tsw_accept_workspace_size() bytes.  Errors as for both. */
int tsw_accept_greedy_penalized(const int32_t* parent, int32_t T, const void* logits, int64_t vocab,
                                int32_t logits_dtype, const int32_t* draft, const int32_t* recent, int64_t n_recent,
                                int32_t window, float theta, int32_t* result, void* workspace,
                                size_t workspace_bytes, tsw_stream_t stream);

/* Moves the accepted path's K and V rows into place for n_layers caches:
 * for k = 1 .. L-1 the row at n_prefix + path[k] is copied to n_prefix + k
 * (row n_prefix + 0, the root, stays); the caller then commits
 * n_prefix + L positions.  k, v: device, layer l at element offset
 * l * layer_stride, each [Hkv][rows][d] with kv_head_stride elements between
 * heads, rows >= n_prefix + T, 16-byte aligned.  result: device, as written
 * by tsw_accept_greedy (read on the device; out-of-range entries are
 * clamped, so no access leaves rows n_prefix .. n_prefix + T - 1).  All
 * source rows are read before any is written.  Errors: TSW_EINVAL,
 * TSW_EUNSUPPORTED (d other than 64/128, dtype), TSW_EHIP. */
int tsw_kv_compact(void* k, void* v, int32_t n_layers, int64_t layer_stride, int32_t Hkv, int32_t d,
                   int32_t dtype, int64_t kv_head_stride, int64_t n_prefix, int32_t T,
                   const int32_t* result, tsw_stream_t stream);

/* ---------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as tsw_tree_attn_verify, same arguments and results, without a
 * workspace argument.  The split partials live in a device array of this
 * library, tsw_noalloc_scratch_bytes() = 32 MiB per GPU, held until the
 * process ends; the call makes no allocation of any kind.  A problem whose
 * tsw_workspace_size() exceeds it returns TSW_ENOSPACE before launching
 * anything.  Every call on one GPU uses that GPU's array: calls that can
 * overlap on one GPU (different streams, different host threads) race on
 * it and must be serialised by the caller; calls on one stream are
 * ordered.  Errors as for tsw_tree_attn_verify.
 * ------------------------------------------------------------------- */
size_t tsw_noalloc_scratch_bytes(void);
int tsw_tree_attn_verify_noalloc(const tsw_attn_desc* desc, const void* q, const void* k, const void* v,
                                 const int32_t* parent, float* o, float* lse, tsw_stream_t stream);

/* ---------------------------------------------------------------------
 * Measurement aid (not a step of the method): the read-stream ceiling of
 * this device for the cache a tsw_tree_attn_verify call with this desc
 * reads.  Streams rows 0 .. n_prefix + T - 1 of every kv head of k and v
 * through the same kind of LDS-DMA ring and grid as the matrix-core split
 * kernel, with no arithmetic, so its rate (2 * Hkv * (n_prefix + T) * d * 2
 * bytes per call) bounds what the split kernel can stream.  bfloat16,
 * d = 128; k and v 16-byte aligned; sink: device memory of at least 64 bytes
 * (never written for real data).  Errors: TSW_EINVAL, TSW_EUNSUPPORTED,
 * TSW_EHIP. */
int tsw_read_stream(const tsw_attn_desc* desc, const void* k, const void* v, unsigned* sink, tsw_stream_t stream);

/* Measurement aid, not a step of the method: the launch floor of the split
 * phase.  Launches a kernel that does nothing on the grid, block size and
 * by-value argument size tsw_tree_attn_verify (n_idx < 0) or
 * tsw_tree_attn_partial (n_idx >= 0) would use for its split kernel, so
 * that a caller can time "empty split + merge" beside the real call.
 * *threads (may be NULL) receives the work-group size.  Errors: as
 * tsw_plan_splits. */
int tsw_launch_floor(const tsw_attn_desc* desc, int64_t n_idx, int32_t* threads, tsw_stream_t stream);

/* Static description of a status code. */
const char* tsw_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* TSW_H */
