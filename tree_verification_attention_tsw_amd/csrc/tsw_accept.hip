// Greedy acceptance of a verified draft tree and compaction of the accepted
// path's K/V rows (gfx950).
//
// After the verification pass the target model's logits at every tree node
// give its most likely next token there; a drafted node is kept when its
// parent is kept and its token equals that prediction at the parent, and the
// longest kept root path becomes the output.  Sources: "TokenSwift - A
// framework for accelerating the generation of ultra-long text" (aiboss88
// project page), technical principles, tree-based multi-candidate token
// verification (the longest valid n-gram is kept, consistent with the target
// model); Tencent Cloud article "90分钟生成10万Token，新框架实现3倍无损加速超长
// 文本生成", 技术原理, parallel-verification figure text (the longest valid
// candidate is selected after checking against the full KV cache).
//
// Kernels:
//   context_penalty one work-group per node: the repetition penalty on the
//                   logits of the tokens in the node's window (in place),
//                   before the argmax when the caller asks for it.
//   argmax_partial  grid (chunks, T): each work-group scans one slice of one
//                   node's logits with 16-byte loads and keeps the largest
//                   value (first index among equals).  HBM-bound.
//   accept_walk     one wavefront (lane = node): folds the slices per node,
//                   then finds the accepted nodes by pointer jumping.
//   kv_compact      grid (kv head, layer, K|V): moves the accepted path's
//                   rows to n_prefix, n_prefix + 1, ...; all sources are read
//                   into LDS before any destination is written, since a
//                   destination row can be the source of an earlier move.
#include <limits.h>

#include "tsw_device.h"
#include "tsw_internal.h"

namespace tsw {

namespace {

// (value, index) with the larger value winning and the lower index breaking
// ties.  An unset pair has index INT_MAX, so any element beats it.
struct Best {
    float v;
    int i;
};

__device__ __forceinline__ Best better(Best a, Best b) {
    if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
    return a;
}

__device__ __forceinline__ Best wave_best(Best x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        Best y;
        y.v = __shfl_xor(x.v, m);
        y.i = __shfl_xor(x.i, m);
        x = better(x, y);
    }
    return x;
}

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(__bf16 x) { return (float)x; }

// Node t's penalty window, oldest first: the last `window` tokens of the
// committed tokens (ending with the root's) followed by the draft tokens on
// the path from the root down to t.  The path's nodes come from the parent
// array in the kernel arguments (scalar reads, no memory round trip); the
// path tokens and this thread's committed tokens are then loaded together,
// so the window costs one memory round trip.  Thread j of the work-group
// gets window entries first + j + 256 * k in tok[k] (-1 past the end).
constexpr int kWinPer = kPenaltyMaxWindow / 256;

struct WindowLds {
    int32_t nodes[64];
    int32_t tok[64];
    int depth;
};

__device__ __forceinline__ void load_window(const int32_t* parent, int32_t window, int64_t n_recent,
                                            const int32_t* __restrict__ recent, const int32_t* __restrict__ draft,
                                            int t, WindowLds& w, int32_t (&tok)[kWinPer]) {
    if (threadIdx.x == 0) {
        int d = 0;
        for (int x = t; x != 0; x = parent[x]) w.nodes[d++] = x;   // parent[x] < x: ends at the root
        w.depth = d;
    }
    __syncthreads();
    const int d = w.depth;
    if ((int)threadIdx.x < d) w.tok[threadIdx.x] = draft[w.nodes[threadIdx.x]];   // deepest first
    const int64_t total = n_recent + d;
    const int64_t first = total - (window < total ? window : total);
#pragma unroll
    for (int k = 0; k < kWinPer; ++k) {
        const int64_t i = first + threadIdx.x + 256 * k;
        tok[k] = i < n_recent && i < total ? recent[i] : -1;
    }
    __syncthreads();                                 // the path tokens are in LDS
#pragma unroll
    for (int k = 0; k < kWinPer; ++k) {
        const int64_t i = first + threadIdx.x + 256 * k;
        if (i >= n_recent && i < total) tok[k] = w.tok[d - 1 - (int)(i - n_recent)];
    }
}

__device__ __forceinline__ float round_as(float x, float) { return x; }
__device__ __forceinline__ float round_as(float x, __bf16) { return (float)(__bf16)x; }   // nearest even

// One slice of one node's logits: the largest value and its first index.
// With PEN the node's contextual penalty is applied on the fly: the window
// tokens that fall in the slice are marked in an LDS bitmap and skipped by
// the scan, and enter instead with their penalised values (formed from the
// logits as given, so a repeated token counts once).  The logits are not
// modified.
template <typename TIN, bool PEN>
__global__ __launch_bounds__(256) void argmax_partial(const AcceptArgs a, const TIN* __restrict__ logits,
                                                      int64_t vocab, int64_t chunk, bool vec_ok,
                                                      const int32_t* __restrict__ draft,
                                                      AcceptPartial* __restrict__ part) {
    constexpr int VEC = 16 / sizeof(TIN);
    const int t = blockIdx.y;
    const int c = blockIdx.x;
    const TIN* row = logits + (int64_t)t * vocab;
    const int64_t start = (int64_t)c * chunk;
    const int64_t end = start + chunk < vocab ? start + chunk : vocab;
    Best b{-INFINITY, INT_MAX};
    __shared__ uint32_t marks[PEN ? kAcceptSliceMax / 32 : 1];
    __shared__ WindowLds wl;
    if constexpr (PEN) {
        const int nw = (int)((end - start + 31) >> 5);
        for (int i = threadIdx.x; i < nw; i += 256) marks[i] = 0u;
        int32_t tok[kWinPer];
        load_window(a.parent, a.window, a.n_recent, a.recent, draft, t, wl, tok);   // barriers inside
#pragma unroll
        for (int k = 0; k < kWinPer; ++k) {
            const int32_t v = tok[k];
            if (v >= start && v < end) {
                const uint32_t off = (uint32_t)(v - start);
                atomicOr(&marks[off >> 5], 1u << (off & 31));
                const float l = widen(row[v]);
                const float p = round_as(l > 0.0f ? __fdiv_rn(l, a.theta) : __fmul_rn(l, a.theta), TIN{});
                b = better(b, Best{p, v});
            }
        }
        __syncthreads();
    }
    auto marked = [&](int64_t i) {
        if constexpr (PEN) {
            const uint32_t off = (uint32_t)(i - start);
            return ((marks[off >> 5] >> (off & 31)) & 1u) != 0u;
        } else {
            return false;
        }
    };
    // the marks of one vector's VEC elements (start is a multiple of 2048 and
    // vectors are VEC-aligned within the slice, so they share one word)
    auto field = [&](int64_t i) -> uint32_t {
        if constexpr (PEN) {
            const uint32_t off = (uint32_t)(i - start);
            return (marks[off >> 5] >> (off & 31)) & ((1u << VEC) - 1u);
        } else {
            return 0u;
        }
    };
    if (vec_ok) {
        // start and the row are 16-byte aligned: whole vectors (four loads in
        // flight per lane), then the tail
        typedef TIN vec_t __attribute__((ext_vector_type(VEC)));
        constexpr int64_t STEP = 256 * VEC;
        const int64_t vend = start + ((end - start) / VEC) * VEC;
        int64_t i = start + (int64_t)threadIdx.x * VEC;
        for (; i + 3 * STEP < vend; i += 4 * STEP) {
            vec_t x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = *(const vec_t*)(row + i + u * STEP);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t f = field(i + u * STEP);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (!((f >> e) & 1u)) b = better(b, Best{widen(x[u][e]), (int)(i + u * STEP + e)});
            }
        }
        for (; i < vend; i += STEP) {
            const vec_t x = *(const vec_t*)(row + i);
            const uint32_t f = field(i);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (!((f >> e) & 1u)) b = better(b, Best{widen(x[e]), (int)(i + e)});
        }
        for (int64_t j = vend + threadIdx.x; j < end; j += 256)
            if (!marked(j)) b = better(b, Best{widen(row[j]), (int)j});
    } else {
        for (int64_t i = start + threadIdx.x; i < end; i += 256)
            if (!marked(i)) b = better(b, Best{widen(row[i]), (int)i});
    }
    b = wave_best(b);
    __shared__ Best wb[4];
    if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = b;
    __syncthreads();
    if (threadIdx.x == 0) {
        Best r = better(better(wb[0], wb[1]), better(wb[2], wb[3]));
        part[(int64_t)t * a.n_chunks + c] = AcceptPartial{r.v, r.i};
    }
}

// One wavefront, lane i = node i.  A node agrees with the target when its
// draft token is the most likely token at its parent; it is accepted when
// every node on its root path agrees, found by pointer jumping (six steps
// cover depth 63).  The deepest accepted node (lowest index among equals)
// is picked by a wave reduction, and its ancestor-or-self bits give the path
// (the node at depth k is path entry k).
__global__ __launch_bounds__(64) void accept_walk(const AcceptArgs a, const AcceptPartial* __restrict__ part,
                                                  const int32_t* __restrict__ draft, int32_t* __restrict__ result) {
    const int t = threadIdx.x;
    const bool live = t < a.T;
    int tok = 0;
    if (live) {
        // the fold is order-free (largest value, lowest index among equal
        // ones; NaN never wins), so the slices' partials are loaded U at a
        // time before they are folded: one memory round trip per U slices
        constexpr int U = 16;
        Best b{-INFINITY, INT_MAX};
        const AcceptPartial* row = part + (int64_t)t * a.n_chunks;
        for (int c0 = 0; c0 < a.n_chunks; c0 += U) {
            AcceptPartial p[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                p[u] = c0 + u < a.n_chunks ? row[c0 + u] : AcceptPartial{-INFINITY, INT_MAX};
#pragma unroll
            for (int u = 0; u < U; ++u) b = better(b, Best{p[u].v, p[u].i});
        }
        // all-NaN rows leave no index: report token 0 (NaN logits are outside
        // the contract)
        tok = b.i == INT_MAX ? 0 : b.i;
        result[2 + a.T + t] = tok;
    }
    const int par = live && t > 0 ? a.parent[t] : 0;
    const int parent_tok = __shfl(tok, par);
    int ok = live && (t == 0 || draft[t] == parent_tok);
    int anc = par;
#pragma unroll
    for (int step = 0; step < 6; ++step) {
        ok = ok & __shfl(ok, anc);
        anc = __shfl(anc, anc);
    }
    const int depth = live ? a.depth[t] : 0;
    // key: deeper first, then lower index; -1 for nodes not accepted
    int key = ok ? (depth << 8) | (255 - t) : -1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) key = max(key, __shfl_xor(key, m));
    const int best = 255 - (key & 255);               // the root is always accepted, so key >= 0
    const int L = (key >> 8) + 1;
    const uint64_t on_path = a.mask[best];
    const int bonus = __shfl(tok, best);
    if (live) {
        if ((on_path >> t) & 1ull) result[2 + depth] = t;
        if (t >= L) result[2 + t] = -1;
    }
    if (t == 0) {
        result[0] = L;
        result[1] = bonus;
    }
}

// One (kv head, layer, K or V) per work-group.  Row bytes RB = d * element
// size (128, 256 or 512), moved in 16-byte pieces.
__global__ __launch_bounds__(256) void kv_compact(const CompactArgs a, const int32_t* __restrict__ result) {
    __shared__ uint4 stage[63 * 32];                 // up to 63 moved rows of <= 512 bytes
    const int head = blockIdx.x;
    const int layer = blockIdx.y;
    char* base = (char*)(blockIdx.z == 0 ? a.k : a.v) + ((int64_t)layer * a.layer_stride +
                                                         (int64_t)head * a.kv_head_stride) * a.esz;
    int L = result[0];
    L = L < 1 ? 1 : (L > a.T ? a.T : L);
    const int pieces = a.row_bytes / 16;
    const int n = (L - 1) * pieces;                  // row 0 (the root) never moves
    for (int e = threadIdx.x; e < n; e += 256) {
        const int k = 1 + e / pieces;
        int src = result[2 + k];
        src = src < 0 ? 0 : (src >= a.T ? a.T - 1 : src);
        stage[e] = *(const uint4*)(base + (a.n_prefix + src) * a.row_bytes + (e % pieces) * 16);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += 256) {
        const int k = 1 + e / pieces;
        *(uint4*)(base + (a.n_prefix + k) * a.row_bytes + (e % pieces) * 16) = stage[e];
    }
}

__device__ __forceinline__ void narrow_store(float* p, float x) { *p = x; }
__device__ __forceinline__ void narrow_store(__bf16* p, float x) { *p = (__bf16)x; }   // nearest even

// One work-group per tree node t.  Its window is the last `window` tokens of
// the committed tokens (ending with the root's) followed by the draft tokens
// on the path from the root down to t, i.e. what sequential generation had
// produced before predicting the token after t.  Every logit the window names
// is read and its penalised value formed before the work-group barrier, and
// only then written, so a token that occurs several times is penalised once
// (its writes all carry the same value).  Ids outside [0, vocab) are skipped.
template <typename TIN>
__global__ __launch_bounds__(256) void context_penalty(const PenaltyArgs a, TIN* __restrict__ logits,
                                                       const int32_t* __restrict__ draft,
                                                       const int32_t* __restrict__ recent) {
    __shared__ WindowLds wl;
    const int t = blockIdx.x;
    TIN* row = logits + (int64_t)t * a.vocab;
    int32_t tok[kWinPer];
    load_window(a.parent, a.window, a.n_recent, recent, draft, t, wl, tok);
    float val[kWinPer];
#pragma unroll
    for (int k = 0; k < kWinPer; ++k) {
        if (tok[k] >= a.vocab) tok[k] = -1;
        val[k] = tok[k] >= 0 ? widen(row[tok[k]]) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kWinPer; ++k)
        val[k] = val[k] > 0.0f ? __fdiv_rn(val[k], a.theta) : __fmul_rn(val[k], a.theta);
    __syncthreads();                                 // every read done before any write
#pragma unroll
    for (int k = 0; k < kWinPer; ++k)
        if (tok[k] >= 0) narrow_store(row + tok[k], val[k]);
}

}  // namespace

hipError_t launch_context_penalty(const PenaltyArgs& a, void* logits, int logits_dtype, const int32_t* draft,
                                  const int32_t* recent, hipStream_t stream) {
    if (logits_dtype == 0)
        hipLaunchKernelGGL(context_penalty<float>, dim3(a.T), dim3(256), 0, stream, a, (float*)logits, draft, recent);
    else
        hipLaunchKernelGGL(context_penalty<__bf16>, dim3(a.T), dim3(256), 0, stream, a, (__bf16*)logits, draft,
                           recent);
    return hipGetLastError();
}

hipError_t launch_accept(const AcceptArgs& a, const void* logits, int logits_dtype, int64_t vocab, int64_t chunk,
                         bool vec_ok, const int32_t* draft, int32_t* result, AcceptPartial* part,
                         hipStream_t stream) {
    const dim3 grid(a.n_chunks, a.T);
    const bool pen = a.window > 0;
#define TSW_ARGMAX(TIN_, PEN_)                                                                                \
    hipLaunchKernelGGL((argmax_partial<TIN_, PEN_>), grid, dim3(256), 0, stream, a, (const TIN_*)logits, vocab, \
                       chunk, vec_ok, draft, part)
    if (logits_dtype == 0) {
        if (pen) TSW_ARGMAX(float, true);
        else TSW_ARGMAX(float, false);
    } else {
        if (pen) TSW_ARGMAX(__bf16, true);
        else TSW_ARGMAX(__bf16, false);
    }
#undef TSW_ARGMAX
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_walk, dim3(1), dim3(64), 0, stream, a, part, draft, result);
    return hipGetLastError();
}

hipError_t launch_kv_compact(const CompactArgs& a, int n_layers, int n_kv_heads, const int32_t* result,
                             hipStream_t stream) {
    hipLaunchKernelGGL(kv_compact, dim3(n_kv_heads, n_layers, 2), dim3(256), 0, stream, a, result);
    return hipGetLastError();
}

}  // namespace tsw
