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
// Two kernels:
//   importance_kernel  grid over key chunks: a work-group takes its chunk
//                      through every kv head in turn (so the per-key sums are
//                      formed in one fixed order, no atomics), a wavefront 16
//                      keys at a time with lane (key, quarter of d).
//   select_kernel      one work-group: radix selection of the r-th largest
//                      importance (four 8-bit passes over the float bits,
//                      which order non-negative floats), then an in-order
//                      compaction that keeps every larger one and the first
//                      ties by position.  Output ascending.
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

// Block-wide exclusive scan of one value per thread (1024 threads); returns
// the exclusive prefix and writes the total to *total.
__device__ int block_scan(int x, int* scratch, int* total) {
    const int t = threadIdx.x;
    scratch[t] = x;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int y = t >= off ? scratch[t - off] : 0;
        __syncthreads();
        scratch[t] += y;
        __syncthreads();
    }
    const int incl = scratch[t];
    *total = scratch[1023];
    __syncthreads();
    return incl - x;
}

__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ imp, int64_t n_prefix, int64_t n_keep,
                                                      int64_t n_out, int32_t* __restrict__ idx) {
    __shared__ int hist[256];
    __shared__ int scratch[1024];
    __shared__ uint32_t s_prefix, s_need;
    const int t = threadIdx.x;
    for (int64_t i = t; i < n_keep; i += 1024) idx[i] = (int32_t)i;
    const int64_t m = n_prefix - n_keep;             // candidates
    const int64_t r = n_out - n_keep;                // to choose among them
    if (r <= 0) return;
    const uint32_t* key = (const uint32_t*)(imp + n_keep);   // non-negative floats order as uint32
    uint32_t prefix = 0, mask = 0, need = (uint32_t)r;
    if (r < m) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            hist[t & 255] = 0;
            __syncthreads();
            for (int64_t i = t; i < m; i += 1024) {
                const uint32_t k = key[i];
                if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
            }
            __syncthreads();
            if (t == 0) {
                uint32_t cum = 0, digit = 0;
                for (int b = 255; b >= 0; --b) {
                    if (cum + hist[b] >= need) {
                        digit = b;
                        break;
                    }
                    cum += hist[b];
                }
                s_need = need - cum;                 // still to take inside this bin
                s_prefix = prefix | (digit << shift);
            }
            __syncthreads();
            prefix = s_prefix;
            need = s_need;
            mask |= 255u << shift;
            __syncthreads();
        }
    } else {
        prefix = 0;                                  // everything is taken: threshold 0,
        need = (uint32_t)m;                          // every tie (all of them) kept
    }
    // In position order: every key above the threshold, and the first `need`
    // keys equal to it.  Each thread owns a contiguous run of candidates.
    const int64_t per = (m + 1023) / 1024;
    const int64_t lo = t * per, hi = lo + per < m ? lo + per : m;
    int gt = 0, eq = 0;
    for (int64_t i = lo; i < hi; ++i) {
        const uint32_t k = key[i];
        gt += k > prefix;
        eq += k == prefix;
    }
    int tot;
    const int gt_before = block_scan(gt, scratch, &tot);
    const int eq_before = block_scan(eq, scratch, &tot);
    int64_t out = n_keep + gt_before + (eq_before < (int)need ? eq_before : (int)need);
    int eq_seen = eq_before;
    for (int64_t i = lo; i < hi; ++i) {
        const uint32_t k = key[i];
        bool take = k > prefix;
        if (k == prefix) {
            take = eq_seen < (int)need;
            ++eq_seen;
        }
        if (take) idx[out++] = (int32_t)(n_keep + i);
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

hipError_t launch_select(const float* imp, int64_t n_prefix, int64_t n_keep, int64_t n_out, int32_t* idx,
                         hipStream_t stream) {
    hipLaunchKernelGGL(select_kernel, dim3(1), dim3(1024), 0, stream, imp, n_prefix, n_keep, n_out, idx);
    return hipGetLastError();
}

}  // namespace tsw
