// Importance of committed KV positions and selection of the draft pass's
// partial cache (gfx950).
//
// The draft pass runs the target model over a partial KV cache that always
// keeps the initial positions and keeps the rest by importance.  Sources:
// "TokenSwift - A framework for accelerating the generation of ultra-long
// text" (aiboss88 project page), technical principles, dynamic KV cache
// update (initial KV kept, the rest ordered by importance); Tencent Cloud
// article "90分钟生成10万Token，新框架实现3倍无损加速超长文本生成", 无损的输出质量
// (the draft model is the target model with a partial KV cache).  The pages
// do not define importance; here it is the attention mass the tree root's
// query heads (node 0, the last committed token) put on each position in the
// verification pass: imp[p] = sum_h exp(scale * q[0][h] . k[g(h)][p] - LSE[0][h]).
//
// Kernels:
//   importance_kernel  grid over key chunks: a work-group takes its chunk
//                      through every kv head in turn (so the per-key sums are
//                      formed in one fixed order, no atomics), a wavefront
//                      holding 4 x 16 keys with lane (key, quarter of d), the
//                      next head's rows loading while one head's are used.
//   select_keep        the kept initial positions; clears the digit totals.
//   importance_from_scores  the same importance from the root-row scores the
//                      verification kernel wrote (K is not read again), with
//                      the first radix pass's digit counts.
//   select_count x4    radix selection of the r-th largest importance: four
//                      8-bit passes over the float bits (which order
//                      non-negative floats), digit counts summed into the
//                      pass's totals; every block re-derives the state of
//                      the earlier passes from those totals, so no launch
//                      needs a host round trip.
//   select_flags       per block: keys above the threshold and equal to it.
//   select_write       the chosen positions in order (every larger key, the
//                      first `need` equal ones), each block offset by the
//                      counts of the blocks before it.  Output ascending.
#include <limits.h>

#include "tsw_device.h"
#include "tsw_internal.h"

namespace tsw {

namespace {

__device__ __forceinline__ float widen_e(float x) { return x; }
__device__ __forceinline__ float widen_e(__bf16 x) { return (float)x; }

template <typename TIN, int D>
__global__ __launch_bounds__(256) void importance_kernel(const SelectArgs a, int chunk, float* __restrict__ imp) {
    constexpr int QD = D / 4;                       // head-dim elements per lane
    constexpr int VEC = 16 / sizeof(TIN);           // elements per 16-byte load
    constexpr int NV = QD / VEC;                    // loads per lane and key
    constexpr int J = kSelectChunk / 64;            // 16-key groups per wave and head
    // bf16 keys: the next kv head's rows are loaded while this one's are used
    constexpr bool PF = sizeof(TIN) == 2;
    typedef TIN vec_t __attribute__((ext_vector_type(VEC)));
    // node 0's query heads (as given: bf16 pairs or floats) and their LSE
    __shared__ TIN qs[kSelectMaxHeads * D];
    __shared__ float ls[kSelectMaxHeads];

    // chunk <= kSelectChunk keys per work-group
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int n = (int)(a.n_prefix - c0 < chunk ? a.n_prefix - c0 : chunk);
    const TIN* q = (const TIN*)a.q;                 // row 0 = node 0
    for (int i = threadIdx.x; i < a.Hq * D; i += 256) qs[i] = q[i];
    for (int i = threadIdx.x; i < a.Hq; i += 256) ls[i] = a.lse[i];
    __syncthreads();

    // lane (li, lj) of wave w holds keys w*16 + j*64 + li (j < J), quarter lj
    // of the head dim; every key's sum over the heads is formed by one lane
    // in head order
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lj = lane >> 4;
    float mine[J];
#pragma unroll
    for (int j = 0; j < J; ++j) mine[j] = 0.0f;
    auto load = [&](int g, vec_t (&x)[J][NV]) {
        const TIN* kg = (const TIN*)a.k + (size_t)g * a.kv_head_stride;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int key = wave * 16 + j * 64 + li;
            const TIN* row = kg + (size_t)(c0 + (key < n ? key : 0)) * D + lj * QD;
#pragma unroll
            for (int v = 0; v < NV; ++v) x[j][v] = *(const vec_t*)(row + v * VEC);
        }
    };
    // one kv head: each query head's quarter is read from LDS once and used
    // for all J key groups; bf16 pairs go through v_dot2_f32_bf16 (products
    // of bf16 values are exact in float32), floats through FMAs
    auto use = [&](int g, const vec_t (&x)[J][NV]) {
        float sum[J];
#pragma unroll
        for (int j = 0; j < J; ++j) sum[j] = 0.0f;
        for (int jj = 0; jj < a.G; ++jj) {
            const int h = g * a.G + jj;
            const float lh = ls[h];
            float dot[J];
            if constexpr (sizeof(TIN) == 2) {
                const bf16x2* qh = (const bf16x2*)(qs + h * D + lj * QD);
                bf16x2 qv[QD / 2];
#pragma unroll
                for (int e = 0; e < QD / 2; ++e) qv[e] = qh[e];
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    float acc = 0.0f;
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int e = 0; e < VEC; e += 2) {
                            const bf16x2 kp = {x[j][v][e], x[j][v][e + 1]};
                            acc = __builtin_amdgcn_fdot2_f32_bf16(kp, qv[(v * VEC + e) / 2], acc, false);
                        }
                    dot[j] = acc;
                }
            } else {
                const float* qh = (const float*)(qs + h * D + lj * QD);
                float qv[QD];
#pragma unroll
                for (int e = 0; e < QD; ++e) qv[e] = qh[e];
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    float acc = 0.0f;
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int e = 0; e < VEC; ++e) acc = fmaf(qv[v * VEC + e], widen_e(x[j][v][e]), acc);
                    dot[j] = acc;
                }
            }
#pragma unroll
            for (int j = 0; j < J; ++j) sum[j] += __expf(quad_sum(dot[j]) * a.scale - lh);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) mine[j] += sum[j];
    };
    if constexpr (PF) {
        vec_t xa[J][NV], xb[J][NV];
        load(0, xa);
        int g = 0;
        for (; g + 1 < a.Hkv; g += 2) {
            load(g + 1, xb);
            use(g, xa);
            if (g + 2 < a.Hkv) load(g + 2, xa);
            use(g + 1, xb);
        }
        if (g < a.Hkv) use(g, xa);
    } else {
        vec_t x[J][NV];
        for (int g = 0; g < a.Hkv; ++g) {
            load(g, x);
            use(g, x);
        }
    }
    if (lj == 0) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int key = wave * 16 + j * 64 + li;
            if (key < n) imp[c0 + key] = mine[j];
        }
    }
}

// Selection state after `passes` radix passes, derived from the digit totals
// of those passes (every work-group derives the same values).  The digit of
// a pass is the one whose count, added to the counts of the larger digits,
// first reaches the number still needed.  Wavefront 0 does it: lane l holds
// digits 4l..4l+3, a shuffle suffix scan over the lanes gives each lane the
// count above its digits, and the one lane whose range holds the crossing
// names the digit.  One barrier publishes the state.
struct SelState {
    uint32_t prefix, mask, need;
};

__device__ SelState derive_state(const uint32_t* __restrict__ totals, int passes, uint32_t r,
                                 uint32_t* out /* LDS [3] */) {
    if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        uint4 v[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            v[p] = p < passes ? *(const uint4*)(totals + p * 256 + 4 * l) : uint4{0u, 0u, 0u, 0u};
        uint32_t prefix = 0u, mask = 0u, need = r;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (p >= passes) break;
            const uint32_t mine = v[p].x + v[p].y + v[p].z + v[p].w;
            uint32_t sfx = mine;                     // sum over lanes >= l
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_down(sfx, off);
                if (l + off < 64) sfx += y;
            }
            // counts above digits 4l+3, 4l+2, 4l+1, 4l
            const uint32_t a3 = sfx - mine, a2 = a3 + v[p].w, a1 = a2 + v[p].z, a0 = a1 + v[p].y;
            int d = -1;
            uint32_t rest = 0u;
            if (a3 < need && need <= a2) { d = 4 * l + 3; rest = need - a3; }
            else if (a2 < need && need <= a1) { d = 4 * l + 2; rest = need - a2; }
            else if (a1 < need && need <= a0) { d = 4 * l + 1; rest = need - a1; }
            else if (a0 < need && need <= a0 + v[p].x) { d = 4 * l; rest = need - a0; }
            const uint64_t found = __builtin_amdgcn_ballot_w64(d >= 0);
            const int src = found ? __builtin_ctzll(found) : 0;   // exactly one lane when need <= candidates
            const uint32_t dig = (uint32_t)__shfl(d, src) & 255u;
            need = (uint32_t)__shfl(rest, src);
            prefix |= dig << (24 - 8 * p);
            mask |= 255u << (24 - 8 * p);
        }
        if (l == 0) {
            out[0] = prefix;
            out[1] = mask;
            out[2] = need;
        }
    }
    __syncthreads();
    return SelState{out[0], out[1], out[2]};
}

// The always-kept initial positions; also clears the digit totals of the
// four passes that follow.
__global__ __launch_bounds__(256) void select_keep(int64_t n_keep, int32_t* __restrict__ idx,
                                                   uint32_t* __restrict__ totals) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_keep) idx[i] = (int32_t)i;
    if (blockIdx.x == 0)
        for (int j = threadIdx.x; j < 4 * 256; j += 256) totals[j] = 0u;
}

// Adds the hitting lanes' digits d to a wave's LDS table: one add when they
// all share a digit (values are often concentrated in a few high digits),
// else one LDS atomic per lane.
__device__ __forceinline__ void wave_count(uint32_t* wt, uint32_t d, bool hit) {
    const uint64_t hits = __builtin_amdgcn_ballot_w64(hit);
    if (hits == 0) return;
    const uint32_t d_first = __shfl(d, __builtin_ctzll(hits));       // the first hitting lane's digit
    const bool same = __builtin_amdgcn_ballot_w64(hit && d != d_first) == 0;
    if (same) {
        if ((threadIdx.x & 63) == 0) wt[d_first] += (uint32_t)__builtin_popcountll(hits);
    } else if (hit) {
        atomicAdd(&wt[d], 1u);
    }
}

// Importance from the root-row scores the verification kernel wrote:
// imp[p] = sum_h 2^(c * s[h][p] - log2(e) * lse[h]) over the query heads in
// order (c = scale * log2(e)), four keys per thread; also idx[p] = p for the
// kept positions p < n_keep.  With totals != nullptr it adds the first radix
// pass's digit counts of the candidates p >= n_keep (the totals were cleared
// by the verification kernel).
__global__ __launch_bounds__(256) void importance_from_scores(const float* __restrict__ root_s, int64_t stride,
                                                              const float* __restrict__ lse, int Hq,
                                                              int64_t n_prefix, float c, int64_t n_keep,
                                                              float* __restrict__ imp,
                                                              uint32_t* __restrict__ totals,
                                                              int32_t* __restrict__ idx) {
    __shared__ float ls[kSelectMaxHeads];
    __shared__ uint32_t wt[4][256];
    const int t = threadIdx.x, w = t >> 6;
    for (int i = t; i < Hq; i += 256) ls[i] = lse[i] * kLog2e;
    for (int i = t; i < 4 * 256; i += 256) (&wt[0][0])[i] = 0;
    __syncthreads();
    // four keys per thread (16-byte loads), eight heads' loads in flight
    const int64_t p0 = ((int64_t)blockIdx.x * 256 + t) * 4;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (p0 + 4 <= n_prefix) {
        const float* src = root_s + p0;
#pragma unroll 8
        for (int h = 0; h < Hq; ++h) {
            const f32x4 x = *(const f32x4*)(src + (size_t)h * stride);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += exp2_fast(fmaf(x[i], c, -ls[h]));
        }
    } else if (p0 < n_prefix) {
        for (int h = 0; h < Hq; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (p0 + i < n_prefix) acc[i] += exp2_fast(fmaf(root_s[(size_t)h * stride + p0 + i], c, -ls[h]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (p0 + i < n_prefix) imp[p0 + i] = acc[i];
        if (p0 + i < n_keep) idx[p0 + i] = (int32_t)(p0 + i);     // the kept initial positions
    }
    if (totals == nullptr) return;                   // uniform
#pragma unroll
    for (int i = 0; i < 4; ++i)
        wave_count(wt[w], __float_as_uint(acc[i]) >> 24, p0 + i >= n_keep && p0 + i < n_prefix);
    __syncthreads();
    const uint32_t cnt = wt[0][t] + wt[1][t] + wt[2][t] + wt[3][t];
    if (cnt) atomicAdd(&totals[t], cnt);
}

// Radix pass `pass` (8-bit digit, high to low) over block blockIdx.x's
// kSelBlock candidates: digit counts of the keys that match the state so
// far, added to the pass's totals (per-wave LDS tables first).
__global__ __launch_bounds__(256) void select_count(const uint32_t* __restrict__ key, int64_t m, uint32_t r, int pass,
                                                    uint32_t* __restrict__ totals) {
    constexpr int RUN = kSelBlock / 256;
    __shared__ uint32_t wt[4][256];
    __shared__ uint32_t st_lds[3];
    const int t = threadIdx.x, w = t >> 6;
    const int64_t base = (int64_t)blockIdx.x * kSelBlock;
    uint32_t k[RUN];                                 // all loads in flight before the state is known
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
        const int64_t i = base + j * 256 + t;
        k[j] = i < m ? key[i] : 0u;
    }
    for (int i = t; i < 4 * 256; i += 256) (&wt[0][0])[i] = 0;
    const SelState st = derive_state(totals, pass, r, st_lds);
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
        const bool hit = base + j * 256 + t < m && (k[j] & st.mask) == st.prefix;
        wave_count(wt[w], (k[j] >> shift) & 255u, hit);
    }
    __syncthreads();
    const uint32_t c = wt[0][t] + wt[1][t] + wt[2][t] + wt[3][t];
    if (c) atomicAdd(&totals[pass * 256 + t], c);
}

// After the four passes: keys above the threshold and keys equal to it, per
// block.
__global__ __launch_bounds__(256) void select_flags(const uint32_t* __restrict__ key, int64_t m, uint32_t r,
                                                    const uint32_t* __restrict__ totals,
                                                    uint32_t* __restrict__ counts) {
    constexpr int RUN = kSelBlock / 256;
    __shared__ uint32_t st_lds[3];
    __shared__ uint32_t red[2][4];
    const int t = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * kSelBlock;
    uint32_t k[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
        const int64_t i = base + j * 256 + t;
        k[j] = i < m ? key[i] : 0u;
    }
    const SelState st = derive_state(totals, 4, r, st_lds);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
        const bool live = base + j * 256 + t < m;
        gt += live && k[j] > st.prefix;
        eq += live && k[j] == st.prefix;
    }
    for (int off = 32; off >= 1; off >>= 1) {
        gt += __shfl_xor(gt, off);
        eq += __shfl_xor(eq, off);
    }
    if ((t & 63) == 0) {
        red[0][t >> 6] = gt;
        red[1][t >> 6] = eq;
    }
    __syncthreads();
    if (t == 0) {
        counts[2 * blockIdx.x] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        counts[2 * blockIdx.x + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    }
}

// Writes the chosen positions in order: a key above the threshold, or equal
// to it while fewer than `need` equal keys come before it.  Thread t of a
// block owns the contiguous run [t*16, t*16+16) of the block.
__global__ __launch_bounds__(256) void select_write(const uint32_t* __restrict__ key, int64_t m, uint32_t r,
                                                    const uint32_t* __restrict__ totals,
                                                    const uint32_t* __restrict__ counts, int64_t n_keep,
                                                    int32_t* __restrict__ idx) {
    constexpr int RUN = kSelBlock / 256;
    __shared__ uint32_t st_lds[3];
    __shared__ uint32_t wsum[2][4];
    __shared__ uint32_t blk_off[2];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t lo = (int64_t)blockIdx.x * kSelBlock + (int64_t)t * RUN;
    uint32_t k[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) k[j] = lo + j < m ? key[lo + j] : 0u;
    const SelState st = derive_state(totals, 4, r, st_lds);
    // counts of the earlier blocks, one block per thread, summed in a wave
    if (t >= 192) {
        uint32_t g = 0, e = 0;
        for (int blk = t - 192; blk < (int)blockIdx.x; blk += 64) {
            g += counts[2 * blk];
            e += counts[2 * blk + 1];
        }
        for (int off = 32; off >= 1; off >>= 1) {
            g += __shfl_xor(g, off);
            e += __shfl_xor(e, off);
        }
        if (t == 192) {
            blk_off[0] = g;
            blk_off[1] = e;
        }
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
        const bool live = lo + j < m;
        gt += live && k[j] > st.prefix;
        eq += live && k[j] == st.prefix;
    }
    // exclusive scans of the per-thread counts across the block: inclusive
    // shuffle scans in each wave, then the totals of the earlier waves
    uint32_t sg = gt, se = eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t yg = __shfl_up(sg, off), ye = __shfl_up(se, off);
        if (lane >= off) {
            sg += yg;
            se += ye;
        }
    }
    if (lane == 63) {
        wsum[0][w] = sg;
        wsum[1][w] = se;
    }
    __syncthreads();
    uint32_t gt_before = blk_off[0] + sg - gt;
    uint32_t eq_before = blk_off[1] + se - eq;
    for (int v = 0; v < w; ++v) {
        gt_before += wsum[0][v];
        eq_before += wsum[1][v];
    }
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
        if (lo + j >= m) break;
        const bool is_gt = k[j] > st.prefix, is_eq = k[j] == st.prefix;
        if (is_gt || (is_eq && eq_before < st.need)) {
            const uint32_t taken_eq = eq_before < st.need ? eq_before : st.need;
            idx[n_keep + gt_before + taken_eq] = (int32_t)(n_keep + lo + j);
        }
        gt_before += is_gt;
        eq_before += is_eq;
    }
}

}  // namespace

hipError_t launch_importance(const SelectArgs& a, float* imp, int cus, hipStream_t stream) {
    if (a.n_prefix == 0) return hipSuccess;
    // two work-groups per CU when the keys allow (a whole round, evenly
    // loaded), at most kSelectChunk keys each, a multiple of 16
    const int64_t want = 2 * (int64_t)(cus > 0 ? cus : 1);
    int64_t chunk = (a.n_prefix + want - 1) / want;
    chunk = (chunk + 15) / 16 * 16;
    if (chunk > kSelectChunk) chunk = kSelectChunk;
    const dim3 grid((unsigned)((a.n_prefix + chunk - 1) / chunk));
    const int c = (int)chunk;
    if (a.dtype == 0) {
        if (a.d == 128) hipLaunchKernelGGL((importance_kernel<float, 128>), grid, dim3(256), 0, stream, a, c, imp);
        else hipLaunchKernelGGL((importance_kernel<float, 64>), grid, dim3(256), 0, stream, a, c, imp);
    } else {
        if (a.d == 128) hipLaunchKernelGGL((importance_kernel<__bf16, 128>), grid, dim3(256), 0, stream, a, c, imp);
        else hipLaunchKernelGGL((importance_kernel<__bf16, 64>), grid, dim3(256), 0, stream, a, c, imp);
    }
    return hipGetLastError();
}

size_t select_scratch_bytes(int64_t n_prefix) {
    const int64_t n_blocks = (n_prefix + kSelBlock - 1) / kSelBlock;
    return (size_t)(4 * 256 + 2 * n_blocks) * sizeof(uint32_t);
}

hipError_t launch_select_keep(int64_t n_keep, int32_t* idx, uint32_t* scratch, hipStream_t stream) {
    hipLaunchKernelGGL(select_keep, dim3((unsigned)(n_keep > 0 ? (n_keep + 255) / 256 : 1)), dim3(256), 0, stream,
                       n_keep, idx, scratch);
    return hipGetLastError();
}

hipError_t launch_select_passes(const float* imp, int64_t n_prefix, int64_t n_keep, int64_t n_out, int32_t* idx,
                                uint32_t* scratch, int first_pass, hipStream_t stream) {
    uint32_t* totals = scratch;                     // [4][256] digit totals
    uint32_t* counts = scratch + 4 * 256;           // [n_blocks][2]
    const int64_t m = n_prefix - n_keep;             // candidates
    const int64_t r = n_out - n_keep;                // to choose among them (r <= m)
    if (m <= 0 || r <= 0) return hipSuccess;
    const int n_blocks = (int)((m + kSelBlock - 1) / kSelBlock);
    const uint32_t* key = (const uint32_t*)(imp + n_keep);     // non-negative floats order as uint32
    hipError_t e;
    for (int pass = first_pass; pass < 4; ++pass) {
        hipLaunchKernelGGL(select_count, dim3(n_blocks), dim3(256), 0, stream, key, m, (uint32_t)r, pass, totals);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(select_flags, dim3(n_blocks), dim3(256), 0, stream, key, m, (uint32_t)r, totals, counts);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_write, dim3(n_blocks), dim3(256), 0, stream, key, m, (uint32_t)r, totals, counts,
                       n_keep, idx);
    return hipGetLastError();
}

hipError_t launch_select(const float* imp, int64_t n_prefix, int64_t n_keep, int64_t n_out, int32_t* idx,
                         uint32_t* scratch, hipStream_t stream) {
    const hipError_t e = launch_select_keep(n_keep, idx, scratch, stream);
    if (e != hipSuccess) return e;
    return launch_select_passes(imp, n_prefix, n_keep, n_out, idx, scratch, 0, stream);
}

hipError_t launch_importance_from_scores(const float* root_s, int64_t stride, const float* lse, int Hq,
                                         int64_t n_prefix, float c, int64_t n_keep, float* imp, uint32_t* totals,
                                         int32_t* idx, hipStream_t stream) {
    if (n_prefix <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((n_prefix + 1023) / 1024);
    hipLaunchKernelGGL(importance_from_scores, dim3(grid), dim3(256), 0, stream, root_s, stride, lse, Hq, n_prefix,
                       c, n_keep, imp, totals, idx);
    return hipGetLastError();
}

}  // namespace tsw
