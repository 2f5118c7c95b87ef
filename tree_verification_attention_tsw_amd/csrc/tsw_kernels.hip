// Tree-verification attention kernels for gfx950 (MI355X, CDNA4).
//
// The step: the T nodes of a candidate token tree attend, under the tree's
// ancestor mask, to the KV cache (all committed positions when verifying,
// an index list of kept positions in the draft pass) plus the tree's own
// rows.  Sources: "TokenSwift - A framework for accelerating the generation
// of ultra-long text" (aiboss88 project page), technical principles (tree
// verification, dynamic KV cache update); Tencent Cloud article
// "90分钟生成10万Token，新框架实现3倍无损加速超长文本生成", 技术原理 figure text
// (verification with the full KV cache) and 无损的输出质量 (draft = target
// model with a partial KV cache).
//
// Work decomposition (split-K flash decoding): work-group (split s, kv head g)
// streams its contiguous slice of the prefix key list once and applies it to
// all M = T * (Hq/Hkv) query rows that share kv head g, so every K/V byte is
// read from HBM once per call.  Each work-group writes a partial result
// (O normalised within the slice, LSE); lse_merge combines the slices.
//
// Two split kernels:
//  * split_mfma: bfloat16, d = 128.  K/V tiles go HBM -> LDS with direct
//    16-byte loads (global_load_lds_dwordx4) through a multi-stage ring;
//    S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16 with key
//    rows on the matrix M axis and query rows on N, so each lane owns one
//    query row: softmax row statistics are per-lane scalars plus two
//    cross-lane steps, and the online-softmax rescale of O is one scalar per
//    lane.  V^T operands come from row-major LDS through ds_read_b64_tr_b16.
//  * split_valu: float32 or bfloat16 inputs, d = 64 or 128, any row count;
//    plain FMA dot products in fp32.  Exact fp32 path for float32 inputs and
//    the fallback for shapes the matrix-core kernel does not cover.
#include <string.h>

#include <type_traits>

#include "tsw_device.h"
#include "tsw_internal.h"

namespace tsw {

// ---------------------------------------------------------------------------
// Vector-ALU split kernel (float32 or bfloat16 inputs, d = 64 or 128)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename TIN, int D, bool GATHER>
__global__ __launch_bounds__(256) void split_valu(const SplitArgs a) {
    constexpr int TK = kValuTile;      // 64 keys per tile
    constexpr int RB = kValuRows;      // 16 query rows per work-group
    constexpr int NC = D / 16;         // output columns per thread
    __shared__ float qs[RB][D];
    __shared__ float ks_[TK][D + 1];
    __shared__ float vs[TK][D];
    __shared__ float ps[RB][TK];

    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const int nrb = (a.M + RB - 1) / RB;
    const int g = blockIdx.y / nrb;
    const int rb = blockIdx.y % nrb;
    const int row = tid >> 4;          // 0..15
    const int col = tid & 15;
    const int r = rb * RB + row;
    const bool row_ok = r < a.M;
    const int t = row_ok ? r / a.G : 0;
    const int h = g * a.G + (row_ok ? r % a.G : 0);
    const uint64_t nm = row_ok ? a.mask[t] : ~0ull;

    const int64_t c0 = (int64_t)split * a.chunk_keys;
    const int64_t c1 = c0 + a.chunk_keys < a.n_keys ? c0 + a.chunk_keys : a.n_keys;
    const int n_pre_tiles = c1 > c0 ? (int)((c1 - c0 + TK - 1) / TK) : 0;
    const int n_tail_tiles = split == a.n_splits - 1 ? (a.T + TK - 1) / TK : 0;
    const int n_tiles = n_pre_tiles + n_tail_tiles;

    const TIN* kb = (const TIN*)a.k + (size_t)g * a.kv_head_stride;
    const TIN* vb = (const TIN*)a.v + (size_t)g * a.kv_head_stride;

    for (int i = tid; i < RB * D; i += 256) {
        const int rr = rb * RB + i / D;
        float x = 0.0f;
        if (rr < a.M) {
            const int tt = rr / a.G, hh = g * a.G + rr % a.G;
            x = to_f32(((const TIN*)a.q)[((size_t)tt * a.Hq + hh) * D + i % D]);
        }
        qs[i / D][i % D] = x;
    }

    float m_run = -INFINITY, l_run = 0.0f;
    float o[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) o[j] = 0.0f;

    for (int tt = 0; tt < n_tiles; ++tt) {
        const bool tail = tt >= n_pre_tiles;
        const int64_t kstart = tail ? (int64_t)(tt - n_pre_tiles) * TK : c0 + (int64_t)tt * TK;
        const int64_t kend = tail ? a.T : c1;
        __syncthreads();
        for (int i = tid; i < TK * D; i += 256) {
            const int kr = i / D, cc = i % D;
            const int64_t key = kstart + kr;
            float kx = 0.0f, vx = 0.0f;
            if (key < kend) {
                const int64_t pos = tail ? a.n_prefix + key : (GATHER ? (int64_t)a.idx[key] : key);
                kx = to_f32(kb[pos * D + cc]);
                vx = to_f32(vb[pos * D + cc]);
            }
            ks_[kr][cc] = kx;
            vs[kr][cc] = vx;
        }
        __syncthreads();

        float s[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kr = col + 16 * i;
            float acc = 0.0f;
#pragma unroll 8
            for (int cc = 0; cc < D; ++cc) acc = fmaf(qs[row][cc], ks_[kr][cc], acc);
            const int64_t key = kstart + kr;
            bool ok = key < kend;
            if (tail) ok = ok && ((nm >> (key & 63)) & 1ull);
            s[i] = ok ? acc * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[i]);
        }
        mx = xor_max(mx, 8);
        mx = xor_max(mx, 4);
        mx = xor_max(mx, 2);
        mx = xor_max(mx, 1);
        const float mnew = fmaxf(m_run, mx);
        const float alpha = mnew == m_run ? 1.0f : exp2f(m_run - mnew);
        const float mu = mnew == -INFINITY ? 0.0f : mnew;
        float lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = exp2f(s[i] - mu);
            lsum += p;
            ps[row][col + 16 * i] = p;
        }
        lsum = xor_sum(lsum, 8);
        lsum = xor_sum(lsum, 4);
        lsum = xor_sum(lsum, 2);
        lsum = xor_sum(lsum, 1);
        l_run = l_run * alpha + lsum;
        m_run = mnew;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NC; ++j) o[j] *= alpha;
        for (int kr = 0; kr < TK; ++kr) {
            const float p = ps[row][kr];
#pragma unroll
            for (int j = 0; j < NC; ++j) o[j] = fmaf(p, vs[kr][col + 16 * j], o[j]);
        }
    }

    if (!row_ok) return;
    const size_t orow = ((size_t)split * a.T + t) * a.Hq + h;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int j = 0; j < NC; ++j) a.part_o[orow * D + col + 16 * j] = o[j] * inv;
    if (col == 0) a.part_lse[orow] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of split results
// ---------------------------------------------------------------------------
// One wavefront per output row (rows grouped by sequence, each sequence with
// its own run of splits): lanes hold the split LSEs (64 at a time),
// wave reductions give the row's LSE, and each lane accumulates d/64
// consecutive columns over the splits with coalesced loads.  The partial
// rows do not depend on the LSEs, so the first CH of them are loaded
// together with the LSEs: a row costs about one memory round trip.  CH (8,
// 16 or 32) is the smallest chunk that holds the split count, so few loads
// repeat a split past the end.

// Output row r from the n_splits partial rows rr of blocks of `stride` rows
// (part_o / part_lse point at the first split of the row's run).
template <int D, int CH>
__device__ __forceinline__ void merge_row(int n_splits, int64_t stride, int64_t rr, int64_t r,
                                          const float* __restrict__ part_o,
                                          const float* __restrict__ part_lse, float* __restrict__ o,
                                          float* __restrict__ lse) {
    constexpr int PER = D / 64;
    using VT = typename std::conditional<PER == 2, float2, float>::type;
    constexpr float kL2e = 1.44269504088896340736f;
    const int lane = threadIdx.x & 63;
    const VT* src = (const VT*)(part_o + rr * D) + lane;
    const int64_t sstride = stride * D / PER;      // VT elements between splits

    // chunk 0 of the partial rows (splits past the end re-read the last one
    // and get weight 0), issued with the first 64 LSEs
    VT x[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) x[j] = src[(int64_t)(j < n_splits ? j : n_splits - 1) * sstride];
    const float ls0 = lane < n_splits ? part_lse[(int64_t)lane * stride + rr] : -INFINITY;

    float mx = ls0;
    for (int s0 = 64; s0 < n_splits; s0 += 64)
        if (s0 + lane < n_splits) mx = fmaxf(mx, part_lse[(int64_t)(s0 + lane) * stride + rr]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = xor_max(mx, m);
    if (mx == -INFINITY) {
#pragma unroll
        for (int e = 0; e < PER; ++e) o[r * D + lane * PER + e] = 0.0f;
        if (lane == 0) lse[r] = -INFINITY;
        return;
    }
    float sum = ls0 == -INFINITY ? 0.0f : exp2f((ls0 - mx) * kL2e);
    for (int s0 = 64; s0 < n_splits; s0 += 64)
        if (s0 + lane < n_splits) {
            const float ls = part_lse[(int64_t)(s0 + lane) * stride + rr];
            sum += ls == -INFINITY ? 0.0f : exp2f((ls - mx) * kL2e);
        }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum = xor_sum(sum, m);
    const float L = mx + logf(sum);

    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    auto fma_row = [&](float wj, const VT& v) {
        if constexpr (PER == 2) {
            acc[0] = fmaf(wj, v.x, acc[0]);
            acc[1] = fmaf(wj, v.y, acc[1]);
        } else {
            acc[0] = fmaf(wj, v, acc[0]);
        }
    };
    for (int s0 = 0; s0 < n_splits; s0 += 64) {
        // weight of split s0 + lane (0 past the end)
        const float ls = s0 == 0 ? ls0 : (s0 + lane < n_splits ? part_lse[(int64_t)(s0 + lane) * stride + rr] : -INFINITY);
        const float wl = ls == -INFINITY ? 0.0f : exp2f((ls - L) * kL2e);
        const int ng = n_splits - s0 < 64 ? n_splits - s0 : 64;
        for (int c0 = 0; c0 < ng; c0 += CH) {
            if (s0 + c0 > 0) {
#pragma unroll
                for (int j = 0; j < CH; ++j) {
                    const int sp = s0 + c0 + j < n_splits ? s0 + c0 + j : n_splits - 1;
                    x[j] = src[(int64_t)sp * sstride];
                }
            }
#pragma unroll
            for (int j = 0; j < CH; ++j) fma_row(__shfl(wl, c0 + j), x[j]);
        }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) o[r * D + lane * PER + e] = acc[e];
    if (lane == 0) lse[r] = L;
}

// One sequence: n_splits blocks of n_rows rows.
template <int D, int CH>
__global__ __launch_bounds__(256) void lse_merge(int n_splits, int64_t n_rows, const float* __restrict__ part_o,
                                                 const float* __restrict__ part_lse, float* __restrict__ o,
                                                 float* __restrict__ lse) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;
    merge_row<D, CH>(n_splits, n_rows, r, r, part_o, part_lse, o, lse);
}

// Head dim 128, two rows per wavefront: 32 lanes per row, four consecutive
// columns per lane, so each load instruction moves the two rows' 1 KB of a
// split's partials (the rows are adjacent and in the same run of splits).
// Lanes of a half hold the split LSEs (32 at a time) and the reductions stay
// inside the half.  Same arithmetic as merge_row, with 32-lane instead of
// 64-lane reduction trees.  rr: the row within its run (blocks of `stride`
// rows from part_o / part_lse); r: the output row; valid: r is a real row
// (the half past an odd row count only loads a valid row and stores nothing).
template <int CH>
__device__ __forceinline__ void merge_pair(int n_splits, int64_t stride, int64_t rr, int64_t r, bool valid,
                                           const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                           float* __restrict__ o, float* __restrict__ lse) {
    constexpr float kL2e = 1.44269504088896340736f;
    const int lane = threadIdx.x & 63, h = lane >> 5, l = lane & 31;
    const f32x4* src = (const f32x4*)(part_o + rr * 128) + l;
    const int64_t sstride = stride * 128 / 4;        // f32x4 elements between splits

    f32x4 x[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) x[j] = src[(int64_t)(j < n_splits ? j : n_splits - 1) * sstride];
    const float ls0 = l < n_splits ? part_lse[(int64_t)l * stride + rr] : -INFINITY;

    float mx = ls0;
    for (int s0 = 32; s0 < n_splits; s0 += 32)
        if (s0 + l < n_splits) mx = fmaxf(mx, part_lse[(int64_t)(s0 + l) * stride + rr]);
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) mx = xor_max(mx, m);
    const bool empty = mx == -INFINITY;
    float sum = ls0 == -INFINITY ? 0.0f : exp2f((ls0 - mx) * kL2e);
    for (int s0 = 32; s0 < n_splits; s0 += 32)
        if (s0 + l < n_splits) {
            const float ls = part_lse[(int64_t)(s0 + l) * stride + rr];
            sum += ls == -INFINITY ? 0.0f : exp2f((ls - mx) * kL2e);
        }
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) sum = xor_sum(sum, m);
    const float L = empty ? -INFINITY : mx + logf(sum);

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < n_splits; s0 += 32) {
        // weight of split s0 + l (0 past the end, and for an empty row)
        const float ls = s0 == 0 ? ls0 : (s0 + l < n_splits ? part_lse[(int64_t)(s0 + l) * stride + rr] : -INFINITY);
        const float wl = (empty || ls == -INFINITY) ? 0.0f : exp2f((ls - L) * kL2e);
        const int ng = n_splits - s0 < 32 ? n_splits - s0 : 32;
        for (int c0 = 0; c0 < ng; c0 += CH) {
            if (s0 + c0 > 0) {
#pragma unroll
                for (int j = 0; j < CH; ++j) {
                    const int sp = s0 + c0 + j < n_splits ? s0 + c0 + j : n_splits - 1;
                    x[j] = src[(int64_t)sp * sstride];
                }
            }
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const float wj = __shfl(wl, (h << 5) + c0 + j);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(wj, x[j][e], acc[e]);
            }
        }
    }
    if (valid) {
        *(f32x4*)(o + r * 128 + 4 * l) = acc;
        if (l == 0) lse[r] = L;
    }
}

// One sequence: n_splits blocks of n_rows rows, two rows per wavefront,
// one wavefront per work-group: the partials are streamed once, and small
// work-groups spread them over every CU (a CU's share of the reads, not the
// arithmetic, sets the time).
template <int CH>
__global__ __launch_bounds__(64) void lse_merge_pairs(int n_splits, int64_t n_rows, const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, float* __restrict__ o,
                                                      float* __restrict__ lse) {
    const int h = (threadIdx.x >> 5) & 1;
    const int64_t r = (int64_t)blockIdx.x * 2 + h;
    if (r - h >= n_rows) return;                     // the whole wave is past the end (uniform)
    const bool valid = r < n_rows;
    const int64_t rl = valid ? r : n_rows - 1;
    merge_pair<CH>(n_splits, n_rows, rl, r, valid, part_o, part_lse, o, lse);
}

// Several sequences with an even number of rows each (so a wavefront's two
// rows share a run of splits), two rows per wavefront, one wavefront per
// work-group.
template <int CH>
__global__ __launch_bounds__(64) void lse_merge_segs_pairs(const MergeSegs segs, int64_t n_rows,
                                                           const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           float* __restrict__ o, float* __restrict__ lse) {
    const int h = (threadIdx.x >> 5) & 1;
    const int64_t r0 = (int64_t)blockIdx.x * 2;
    if (r0 >= n_rows) return;                        // uniform
    const int64_t r = r0 + h;                        // r0 even, rows_per_seg even: same run
    const int seg = (int)((uint32_t)r0 / (uint32_t)segs.rows_per_seg);
    const int64_t rr = r - (int64_t)seg * segs.rows_per_seg;
    const int64_t first = (int64_t)segs.base[seg] * segs.rows_per_seg;
    merge_pair<CH>(segs.base[seg + 1] - segs.base[seg], segs.rows_per_seg, rr, r, r < n_rows, part_o + first * 128,
                   part_lse + first, o, lse);
}

// Several sequences, each with its own run of splits of rows_per_seg rows.
template <int D, int CH>
__global__ __launch_bounds__(256) void lse_merge_segs(const MergeSegs segs, int64_t n_rows,
                                                      const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, float* __restrict__ o,
                                                      float* __restrict__ lse) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;
    const int seg = (int)((uint32_t)r / (uint32_t)segs.rows_per_seg);
    const int64_t rr = r - (int64_t)seg * segs.rows_per_seg;
    const int64_t first = (int64_t)segs.base[seg] * segs.rows_per_seg;
    merge_row<D, CH>(segs.base[seg + 1] - segs.base[seg], segs.rows_per_seg, rr, r, part_o + first * D, part_lse + first,
                 o, lse);
}

// Any head dim: one thread per output element (used for d other than 64/128).
__global__ __launch_bounds__(256) void lse_merge_generic(int n_splits, int64_t n_rows, int d,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse,
                                                         float* __restrict__ o, float* __restrict__ lse) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n_rows * d) return;
    const int64_t r = e / d;
    const int cc = (int)(e % d);
    constexpr float kLog2e = 1.44269504088896340736f;
    float mx = -INFINITY;
    for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, part_lse[s * n_rows + r]);
    if (mx == -INFINITY) {
        o[e] = 0.0f;
        if (cc == 0) lse[r] = -INFINITY;
        return;
    }
    float sum = 0.0f;
    for (int s = 0; s < n_splits; ++s) {
        const float ls = part_lse[s * n_rows + r];
        if (ls != -INFINITY) sum += exp2f((ls - mx) * kLog2e);
    }
    const float L = mx + logf(sum);
    float acc = 0.0f;
    for (int s = 0; s < n_splits; ++s) {
        const float ls = part_lse[s * n_rows + r];
        if (ls == -INFINITY) continue;
        acc = fmaf(exp2f((ls - L) * kLog2e), part_o[(s * n_rows + r) * d + cc], acc);
    }
    o[e] = acc;
    if (cc == 0) lse[r] = L;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename TIN, int D>
static hipError_t launch_valu_t(bool gather, const SplitArgs& a, int n_kv_heads, hipStream_t stream) {
    const int nrb = (a.M + kValuRows - 1) / kValuRows;
    const dim3 grid(a.n_splits, n_kv_heads * nrb);
    if (gather) hipLaunchKernelGGL((split_valu<TIN, D, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((split_valu<TIN, D, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_split_valu(int dtype, int d, bool gather, const SplitArgs& a, int n_kv_heads,
                             hipStream_t stream) {
    if (dtype == 0 && d == 64) return launch_valu_t<float, 64>(gather, a, n_kv_heads, stream);
    if (dtype == 0 && d == 128) return launch_valu_t<float, 128>(gather, a, n_kv_heads, stream);
    if (dtype == 1 && d == 64) return launch_valu_t<__bf16, 64>(gather, a, n_kv_heads, stream);
    if (dtype == 1 && d == 128) return launch_valu_t<__bf16, 128>(gather, a, n_kv_heads, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_lse_merge_segs(const MergeSegs& segs, int64_t n_rows, const float* part_o,
                                 const float* part_lse, float* o, float* lse, hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_rows + 3) / 4));
    int most = 1;
    for (int b = 0; b < segs.n_seg; ++b)
        most = segs.base[b + 1] - segs.base[b] > most ? segs.base[b + 1] - segs.base[b] : most;
    // two rows per wavefront when a wavefront's rows always share a run
    // (even rows per sequence) and the 16-byte pieces are aligned
    if (segs.rows_per_seg % 2 == 0 && (((uintptr_t)part_o | (uintptr_t)o) & 15) == 0) {
        const dim3 pgrid((unsigned)((n_rows + 1) / 2));
        if (most <= 8)
            hipLaunchKernelGGL((lse_merge_segs_pairs<8>), pgrid, dim3(64), 0, stream, segs, n_rows, part_o, part_lse,
                               o, lse);
        else if (most <= 16)
            hipLaunchKernelGGL((lse_merge_segs_pairs<16>), pgrid, dim3(64), 0, stream, segs, n_rows, part_o,
                               part_lse, o, lse);
        else
            hipLaunchKernelGGL((lse_merge_segs_pairs<32>), pgrid, dim3(64), 0, stream, segs, n_rows, part_o,
                               part_lse, o, lse);
        return hipGetLastError();
    }
    if (most <= 8)
        hipLaunchKernelGGL((lse_merge_segs<128, 8>), grid, dim3(256), 0, stream, segs, n_rows, part_o, part_lse, o, lse);
    else if (most <= 16)
        hipLaunchKernelGGL((lse_merge_segs<128, 16>), grid, dim3(256), 0, stream, segs, n_rows, part_o, part_lse, o,
                           lse);
    else
        hipLaunchKernelGGL((lse_merge_segs<128, 32>), grid, dim3(256), 0, stream, segs, n_rows, part_o, part_lse, o,
                           lse);
    return hipGetLastError();
}

hipError_t launch_lse_merge(int n_splits, int64_t n_rows, int d, const float* part_o,
                            const float* part_lse, float* o, float* lse, hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    if (d == 128 || d == 64) {
        const dim3 grid((unsigned)((n_rows + 3) / 4));
#define TSW_MERGE(D_, CH_) \
    hipLaunchKernelGGL((lse_merge<D_, CH_>), grid, dim3(256), 0, stream, n_splits, n_rows, part_o, part_lse, o, lse)
        // the paired kernel moves 16-byte pieces: partials and output must
        // be 16-byte aligned (any alignment takes the row-per-wave kernel)
        const bool aligned16 = (((uintptr_t)part_o | (uintptr_t)o) & 15) == 0;
        if (d == 128 && aligned16) {
            const dim3 pgrid((unsigned)((n_rows + 1) / 2));
#define TSW_MERGE_PAIRS(CH_) \
    hipLaunchKernelGGL((lse_merge_pairs<CH_>), pgrid, dim3(64), 0, stream, n_splits, n_rows, part_o, part_lse, o, lse)
            if (n_splits <= 8) TSW_MERGE_PAIRS(8);
            else if (n_splits <= 16) TSW_MERGE_PAIRS(16);
            else TSW_MERGE_PAIRS(32);
#undef TSW_MERGE_PAIRS
        } else if (d == 128) {
            if (n_splits <= 8) TSW_MERGE(128, 8);
            else if (n_splits <= 16) TSW_MERGE(128, 16);
            else TSW_MERGE(128, 32);
        } else {
            if (n_splits <= 8) TSW_MERGE(64, 8);
            else if (n_splits <= 16) TSW_MERGE(64, 16);
            else TSW_MERGE(64, 32);
        }
#undef TSW_MERGE
        return hipGetLastError();
    }
    const int64_t n = n_rows * d;
    const dim3 grid((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(lse_merge_generic, grid, dim3(256), 0, stream, n_splits, n_rows, d, part_o, part_lse, o, lse);
    return hipGetLastError();
}

}  // namespace tsw
