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
//                      formed in one fixed order, no atomics), a wavefront 16
//                      keys at a time with lane (key, quarter of d).
//   select_keep        the kept initial positions; clears the digit totals.
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
__global__ __launch_bounds__(256) void importance_kernel(const SelectArgs a, float* __restrict__ imp) {
    constexpr int QD = D / 4;                       // head-dim elements per lane
    constexpr int VEC = 16 / sizeof(TIN);           // elements per 16-byte load
    typedef TIN vec_t __attribute__((ext_vector_type(VEC)));
    __shared__ float qs[kSelectMaxHeads * D];       // node 0's query heads
    __shared__ float ls[kSelectMaxHeads];           // and their LSE
    __shared__ float acc[kSelectChunk];             // per-key sums over heads

    const int64_t c0 = (int64_t)blockIdx.x * kSelectChunk;
    const int n = (int)(a.n_prefix - c0 < kSelectChunk ? a.n_prefix - c0 : kSelectChunk);
    const TIN* q = (const TIN*)a.q;                 // row 0 = node 0
    for (int i = threadIdx.x; i < a.Hq * D; i += 256) qs[i] = widen_e(q[i]);
    for (int i = threadIdx.x; i < a.Hq; i += 256) ls[i] = a.lse[i];
    for (int i = threadIdx.x; i < kSelectChunk; i += 256) acc[i] = 0.0f;
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lj = lane >> 4;
    for (int g = 0; g < a.Hkv; ++g) {
        const TIN* kg = (const TIN*)a.k + (size_t)g * a.kv_head_stride;
        for (int base = wave * 16; base < n; base += 64) {
            const int key = base + li;
            const bool ok = key < n;
            const TIN* row = kg + (size_t)(c0 + (ok ? key : 0)) * D + lj * QD;
            float kv[QD];
#pragma unroll
            for (int v = 0; v < QD / VEC; ++v) {
                const vec_t x = *(const vec_t*)(row + v * VEC);
#pragma unroll
                for (int e = 0; e < VEC; ++e) kv[v * VEC + e] = widen_e(x[e]);
            }
            float sum = 0.0f;
            for (int j = 0; j < a.G; ++j) {
                const int h = g * a.G + j;
                const float* qh = qs + h * D + lj * QD;
                float dot = 0.0f;
#pragma unroll
                for (int e = 0; e < QD; ++e) dot = fmaf(qh[e], kv[e], dot);
                dot = quad_sum(dot);
                sum += __expf(dot * a.scale - ls[h]);
            }
            if (ok && lj == 0) acc[key] += sum;
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < n; i += 256) imp[c0 + i] = acc[i];
}

// Selection state after `passes` radix passes, derived from the digit totals
// of those passes (every work-group derives the same values).  The digit of
// a pass is the one whose count, added to the counts of the larger digits,
// first reaches the number still needed: a suffix scan over the 256 digits,
// one digit per thread.
struct SelState {
    uint32_t prefix, mask, need;
};

__device__ SelState derive_state(const uint32_t* __restrict__ totals, int passes, uint32_t r,
                                 uint32_t* sfx /* LDS [256] */, uint32_t* bcast /* LDS [2] */) {
    SelState st{0u, 0u, r};
    const int t = threadIdx.x;
    uint32_t mine[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) mine[p] = p < passes ? totals[p * 256 + t] : 0u;   // one round trip
    for (int p = 0; p < passes; ++p) {
        // inclusive suffix sums: sfx[d] = sum of totals[d' >= d]
        sfx[t] = mine[p];
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const uint32_t y = t + off < 256 ? sfx[t + off] : 0u;
            __syncthreads();
            sfx[t] += y;
            __syncthreads();
        }
        const uint32_t above = sfx[t] - mine[p];     // keys in larger digits
        if (above < st.need && st.need <= sfx[t]) {
            bcast[0] = (uint32_t)t;
            bcast[1] = st.need - above;              // still to take inside this digit
        }
        __syncthreads();
        st.prefix |= bcast[0] << (24 - 8 * p);
        st.mask |= 255u << (24 - 8 * p);
        st.need = bcast[1];
        __syncthreads();
    }
    return st;
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

// Radix pass `pass` (8-bit digit, high to low) over block blockIdx.x's
// kSelBlock candidates: digit counts of the keys that match the state so
// far, added to the pass's totals.  Per-wave LDS tables; a wave whose hitting
// lanes share a digit adds once (values are often concentrated in the high
// digits).
__global__ __launch_bounds__(256) void select_count(const uint32_t* __restrict__ key, int64_t m, uint32_t r, int pass,
                                                    uint32_t* __restrict__ totals) {
    __shared__ uint32_t wt[4][256];
    __shared__ uint32_t sfx[256];
    __shared__ uint32_t bcast[2];
    const int t = threadIdx.x, w = t >> 6;
    for (int i = t; i < 4 * 256; i += 256) (&wt[0][0])[i] = 0;
    const SelState st = derive_state(totals, pass, r, sfx, bcast);
    const int shift = 24 - 8 * pass;
    const int64_t base = (int64_t)blockIdx.x * kSelBlock;
    for (int j = 0; j < kSelBlock / 256; ++j) {
        const int64_t i = base + j * 256 + t;
        const bool live = i < m;
        const uint32_t k = live ? key[i] : 0u;
        const bool hit = live && (k & st.mask) == st.prefix;
        const uint32_t d = (k >> shift) & 255u;
        const uint64_t hits = __builtin_amdgcn_ballot_w64(hit);
        if (hits == 0) continue;
        const uint32_t d_first = __shfl(d, __builtin_ctzll(hits));       // the first hitting lane's digit
        const bool same = __builtin_amdgcn_ballot_w64(hit && d != d_first) == 0;
        if (same) {
            if ((t & 63) == 0) wt[w][d_first] += (uint32_t)__builtin_popcountll(hits);
        } else if (hit) {
            atomicAdd(&wt[w][d], 1u);
        }
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
    __shared__ uint32_t sfx[256];
    __shared__ uint32_t bcast[2];
    __shared__ uint32_t red[2][4];
    const int t = threadIdx.x;
    const SelState st = derive_state(totals, 4, r, sfx, bcast);
    const int64_t base = (int64_t)blockIdx.x * kSelBlock;
    uint32_t gt = 0, eq = 0;
    for (int j = 0; j < kSelBlock / 256; ++j) {
        const int64_t i = base + j * 256 + t;
        if (i < m) {
            const uint32_t k = key[i];
            gt += k > st.prefix;
            eq += k == st.prefix;
        }
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
    __shared__ uint32_t sfx[256];
    __shared__ uint32_t bcast[2];
    __shared__ uint32_t scan[2][256];
    __shared__ uint32_t blk_off[2];
    const int t = threadIdx.x;
    const SelState st = derive_state(totals, 4, r, sfx, bcast);
    // counts of the earlier blocks, one block per thread, summed in a wave
    if (t < 64) {
        uint32_t g = 0, e = 0;
        for (int blk = t; blk < (int)blockIdx.x; blk += 64) {
            g += counts[2 * blk];
            e += counts[2 * blk + 1];
        }
        for (int off = 32; off >= 1; off >>= 1) {
            g += __shfl_xor(g, off);
            e += __shfl_xor(e, off);
        }
        if (t == 0) {
            blk_off[0] = g;
            blk_off[1] = e;
        }
    }
    const int64_t lo = (int64_t)blockIdx.x * kSelBlock + (int64_t)t * RUN;
    uint32_t k[RUN];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
        const bool live = lo + j < m;
        k[j] = live ? key[lo + j] : 0u;
        gt += live && k[j] > st.prefix;
        eq += live && k[j] == st.prefix;
    }
    // exclusive scans of the per-thread counts across the block
    scan[0][t] = gt;
    scan[1][t] = eq;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const uint32_t a0 = t >= off ? scan[0][t - off] : 0u;
        const uint32_t a1 = t >= off ? scan[1][t - off] : 0u;
        __syncthreads();
        scan[0][t] += a0;
        scan[1][t] += a1;
        __syncthreads();
    }
    uint32_t gt_before = blk_off[0] + scan[0][t] - gt;
    uint32_t eq_before = blk_off[1] + scan[1][t] - eq;
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

hipError_t launch_importance(const SelectArgs& a, float* imp, hipStream_t stream) {
    const dim3 grid((unsigned)((a.n_prefix + kSelectChunk - 1) / kSelectChunk));
    if (a.n_prefix == 0) return hipSuccess;
    if (a.dtype == 0) {
        if (a.d == 128) hipLaunchKernelGGL((importance_kernel<float, 128>), grid, dim3(256), 0, stream, a, imp);
        else hipLaunchKernelGGL((importance_kernel<float, 64>), grid, dim3(256), 0, stream, a, imp);
    } else {
        if (a.d == 128) hipLaunchKernelGGL((importance_kernel<__bf16, 128>), grid, dim3(256), 0, stream, a, imp);
        else hipLaunchKernelGGL((importance_kernel<__bf16, 64>), grid, dim3(256), 0, stream, a, imp);
    }
    return hipGetLastError();
}

size_t select_scratch_bytes(int64_t n_prefix) {
    const int64_t n_blocks = (n_prefix + kSelBlock - 1) / kSelBlock;
    return (size_t)(4 * 256 + 2 * n_blocks) * sizeof(uint32_t);
}

hipError_t launch_select(const float* imp, int64_t n_prefix, int64_t n_keep, int64_t n_out, int32_t* idx,
                         uint32_t* scratch, hipStream_t stream) {
    uint32_t* totals = scratch;                     // [4][256] digit totals
    uint32_t* counts = scratch + 4 * 256;           // [n_blocks][2]
    hipLaunchKernelGGL(select_keep, dim3((unsigned)(n_keep > 0 ? (n_keep + 255) / 256 : 1)), dim3(256), 0, stream,
                       n_keep, idx, totals);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t m = n_prefix - n_keep;             // candidates
    const int64_t r = n_out - n_keep;                // to choose among them (r <= m)
    if (m <= 0 || r <= 0) return hipSuccess;
    const int n_blocks = (int)((m + kSelBlock - 1) / kSelBlock);
    const uint32_t* key = (const uint32_t*)(imp + n_keep);     // non-negative floats order as uint32
    for (int pass = 0; pass < 4; ++pass) {
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

}  // namespace tsw
