/*
 * tsw_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, float64 CPU statement of what tree-verification attention
 * computes.  It exists so that the GPU library can be checked against an
 * independent implementation.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Sources (page title, then the part of the page):
 *  [P2-tree]  "TokenSwift - A framework for accelerating the generation of
 *             ultra-long text" (aiboss88 project page), technical principles,
 *             tree-based multi-candidate token verification: candidate tokens
 *             form a tree, are verified in parallel with tree-structured
 *             attention, and the result must equal the target model's own
 *             prediction (lossless).
 *  [P3-verify] "90分钟生成10万Token，新框架实现3倍无损加速超长文本生成" (Tencent
 *             Cloud article), the figure description under 技术原理: candidate
 *             sequences are fed to the model together with the FULL KV cache
 *             for verification; tree-based attention over a token tree yields
 *             several candidate sequences at once.
 *  [P3-lossless] same article, 优势与特点 / 无损的输出质量: the draft model is the
 *             target model itself with only a PARTIAL KV cache.
 *  [P2-kv]    aiboss88 page, technical principles, dynamic KV cache update:
 *             the initial KV entries are always kept, later ones are replaced
 *             according to token importance.
 *  [P4-tree]  "From Hours to Minutes: Lossless Acceleration of Ultra Long
 *             Sequence Generation up to 100K Tokens" (arxivlens summary),
 *             Technical Contribution: the tree is a simple 3-ary tree.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - the tree's own K/V rows sit in the cache right after the committed
 *    prefix, node j at position n_prefix + j;
 *  - a node attends to itself and to every ancestor (ancestor-or-self);
 *  - parent[0] = -1 and 0 <= parent[i] < i for i >= 1;
 *  - grouped-query heads map to kv head h / (Hq / Hkv);
 *  - scores are scale * (q . k); LSE is the natural log of the sum of
 *    exp(score); O and LSE are produced for every (node, query head).
 *
 * What is computed, for node i and query head h (g = kv head of h):
 *    S(i)   = P  u  { n_prefix + j : j is i or an ancestor of i }
 *             P = {0 .. n_prefix-1} (verify) or the index list (partial)
 *    s_p    = scale * sum_c Q[i][h][c] * K[g][p][c]          for p in S(i)
 *    O[i][h][c] = sum_p exp(s_p) V[g][p][c] / sum_p exp(s_p)
 *    LSE[i][h]  = log(sum_p exp(s_p))
 * The maximum score is subtracted before exponentiating; that changes only
 * rounding, not the value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EBADTREE -2
#define ORACLE_EINVAL -1

/* Inputs arrive either as IEEE float32 or as bfloat16 bit patterns.  A
 * bfloat16 value is the upper half of the float32 with the same bits, so the
 * widening below is exact. */
static double load_elem(const void* base, int dtype, int64_t i)
{
    if (dtype == 0) {
        return (double)((const float*)base)[i];
    } else {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

/* Checks the tree encoding: one root at index 0, every other node names an
 * earlier node as its parent. */
static int tree_is_valid(const int32_t* parent, int32_t T)
{
    if (T < 1) return 0;
    if (parent[0] != -1) return 0;
    for (int32_t i = 1; i < T; ++i)
        if (parent[i] < 0 || parent[i] >= i) return 0;
    return 1;
}

/* Ancestor-or-self set of node i as a list, found by walking parent links
 * up to the root.  Returns the list length (depth + 1). */
static int32_t ancestors_or_self(const int32_t* parent, int32_t i, int32_t* out)
{
    int32_t n = 0;
    for (int32_t a = i; a != -1; a = parent[a]) out[n++] = a;
    return n;
}

/* Tree mask: bit j of mask[i] is set when node j is node i or one of its
 * ancestors; depth[i] is the number of edges from the root.  Supports up to
 * 64 nodes (one 64-bit word per node). */
int oracle_mask_build(const int32_t* parent, int32_t T, uint64_t* mask, int32_t* depth)
{
    if (T < 1 || T > 64 || !parent || !mask) return ORACLE_EINVAL;
    if (!tree_is_valid(parent, T)) return ORACLE_EBADTREE;
    int32_t anc[64];
    for (int32_t i = 0; i < T; ++i) {
        int32_t n = ancestors_or_self(parent, i, anc);
        uint64_t m = 0;
        for (int32_t a = 0; a < n; ++a) m |= (uint64_t)1 << anc[a];
        mask[i] = m;
        if (depth) depth[i] = n - 1;
    }
    return ORACLE_OK;
}

/* One output row: node i, query head h.  keys[] lists the cache positions
 * this node may see (prefix part then its ancestor-or-self tree rows). */
static void attend_row(int32_t i, int32_t h, int32_t Hq, int32_t d, int32_t G,
                       int dtype, const void* q, const void* k, const void* v,
                       int64_t kv_head_stride, const int64_t* keys, int64_t n_keys,
                       double scale, double* o_row, double* lse_out, double* s)
{
    const int32_t g = h / G;
    const int64_t q_off = ((int64_t)i * Hq + h) * d;
    const int64_t kv_off = (int64_t)g * kv_head_stride;

    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j) {
        double acc = 0.0;
        const int64_t kr = kv_off + keys[j] * d;
        for (int32_t c = 0; c < d; ++c)
            acc += load_elem(q, dtype, q_off + c) * load_elem(k, dtype, kr + c);
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int32_t c = 0; c < d; ++c) o_row[c] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        const int64_t vr = kv_off + keys[j] * d;
        for (int32_t c = 0; c < d; ++c) o_row[c] += s[j] * load_elem(v, dtype, vr + c);
    }
    for (int32_t c = 0; c < d; ++c) o_row[c] /= l;
    *lse_out = m + log(l);
}

/*
 * Tree attention, verify (idx == NULL: prefix = all of 0..n_prefix-1) or
 * partial (prefix = idx[0..n_idx-1], positions below n_prefix).
 *
 * Layouts: q [T][Hq][d]; k, v [Hkv][*][d] with kv_head_stride elements
 * between heads (>= (n_prefix + T) * d); dtype 0 = float32, 1 = bfloat16.
 *
 * rows: NULL computes every (node, head) row into o[T*Hq][d], lse[T*Hq].
 * Otherwise rows[r] = node * Hq + head for r < n_rows and the results go to
 * o[r][d], lse[r] in list order (for sampled checks of large cases).
 *
 * nthreads: OpenMP threads over rows (rows are independent); <= 0 means one.
 */
int oracle_tree_attn(int32_t T, int32_t Hq, int32_t Hkv, int32_t d, int64_t n_prefix,
                     int32_t dtype, const void* q, const void* k, const void* v,
                     int64_t kv_head_stride, const int32_t* parent,
                     const int32_t* idx, int64_t n_idx, double scale,
                     const int32_t* rows, int64_t n_rows,
                     double* o, double* lse, int32_t nthreads)
{
    if (T < 1 || T > 64 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0) return ORACLE_EINVAL;
    if (n_prefix < 0 || (dtype != 0 && dtype != 1)) return ORACLE_EINVAL;
    if (!q || !k || !v || !parent || !o || !lse) return ORACLE_EINVAL;
    if (kv_head_stride < (n_prefix + T) * (int64_t)d) return ORACLE_EINVAL;
    if (!tree_is_valid(parent, T)) return ORACLE_EBADTREE;
    if (idx) {
        if (n_idx < 0) return ORACLE_EINVAL;
        for (int64_t j = 0; j < n_idx; ++j)
            if (idx[j] < 0 || idx[j] >= n_prefix || (j > 0 && idx[j] <= idx[j - 1]))
                return ORACLE_EINVAL;
    }
    const int32_t G = Hq / Hkv;
    const int64_t n_pre = idx ? n_idx : n_prefix;
    const int64_t total_rows = rows ? n_rows : (int64_t)T * Hq;
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= T * Hq) return ORACLE_EINVAL;

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < total_rows; ++r) {
        const int32_t flat = rows ? rows[r] : (int32_t)r;
        const int32_t i = flat / Hq, h = flat % Hq;
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_pre + T));
        double* s = (double*)malloc(sizeof(double) * (size_t)(n_pre + T));
        if (!keys || !s) {
            free(keys);
            free(s);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        int64_t n = 0;
        for (int64_t j = 0; j < n_pre; ++j) keys[n++] = idx ? (int64_t)idx[j] : j;
        int32_t anc[64];
        int32_t na = ancestors_or_self(parent, i, anc);
        for (int32_t a = 0; a < na; ++a) keys[n++] = n_prefix + anc[a];
        attend_row(i, h, Hq, d, G, dtype, q, k, v, kv_head_stride, keys, n, scale,
                   o + r * d, lse + r, s);
        free(keys);
        free(s);
    }
    return bad ? ORACLE_EINVAL : ORACLE_OK;
}

/* Combines attention results computed over disjoint key subsets: given
 * normalised outputs O_s and log-sum-exps L_s of n_splits parts, the
 * attention over the union is O = sum_s exp(L_s - L) O_s with
 * L = log(sum_s exp(L_s)).  Parts with L_s = -inf are empty and contribute
 * nothing.  part_o [n_splits][n_rows][d], part_lse [n_splits][n_rows]. */
int oracle_lse_merge(int32_t n_splits, int64_t n_rows, int32_t d, const double* part_o,
                     const double* part_lse, double* o, double* lse)
{
    if (n_splits < 1 || n_rows < 0 || d < 1) return ORACLE_EINVAL;
    for (int64_t r = 0; r < n_rows; ++r) {
        double m = -INFINITY;
        for (int32_t s = 0; s < n_splits; ++s)
            if (part_lse[s * n_rows + r] > m) m = part_lse[s * n_rows + r];
        double sum = 0.0;
        for (int32_t s = 0; s < n_splits; ++s)
            if (part_lse[s * n_rows + r] != -INFINITY) sum += exp(part_lse[s * n_rows + r] - m);
        const double L = (m == -INFINITY) ? -INFINITY : m + log(sum);
        for (int32_t c = 0; c < d; ++c) o[r * d + c] = 0.0;
        for (int32_t s = 0; s < n_splits; ++s) {
            const double ls = part_lse[s * n_rows + r];
            if (ls == -INFINITY) continue;
            const double w = exp(ls - L);
            for (int32_t c = 0; c < d; ++c) o[r * d + c] += w * part_o[(s * n_rows + r) * d + c];
        }
        lse[r] = L;
    }
    return ORACLE_OK;
}
