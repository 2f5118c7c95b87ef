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
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tsw_internal.h"

namespace tsw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLn2 = 0.693147180559945309417f;
// Lazy rescale threshold (log2 units): the running maximum is only raised
// when a new score exceeds it by more than this, so exponentials stay below
// 2^8 and the O accumulators are rescaled rarely.
constexpr float kRescaleTau = 8.0f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m)); }
__device__ __forceinline__ float xor_sum(float x, int m) { return x + __shfl_xor(x, m); }

// 16-byte chunk swizzle of a 256-byte LDS row.  Logical chunk c of tile row r
// lives in physical slot c ^ swz(r).  For any 8 (and 16) consecutive aligned
// rows the slots of one logical chunk are all different, and for any 4
// (and 8) consecutive aligned rows the chunk pairs {2b, 2b+1} land in
// different slot pairs, so both the K operand reads (one chunk of 16 rows)
// and the transposed V reads (two chunks of 4 rows per 16 lanes) are free of
// bank conflicts whether the LDS serves 128 or 256 bytes per clock.
__device__ __forceinline__ int swz(int r) { return ((2 * (r & 7)) | ((r >> 2) & 1)) ^ ((r >> 3) & 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Work-group barrier that does not wait for outstanding LDS-DMA loads (the
// pipeline waits for exactly the tiles it needs with wait_vmcnt).  Pending
// LDS reads are drained first so a stage is never overwritten under a read.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Matrix-core split kernel (bfloat16, d = 128)
// ---------------------------------------------------------------------------
template <int WAVES, int R, int NB>
struct MfmaShape {
    static constexpr int KS = WAVES / R;                   // 32-key sub-tiles per tile
    static constexpr int TK = 32 * KS;                     // keys per tile
    static constexpr int ROWB = 256;                       // bytes per K or V row (128 bf16)
    static constexpr int STAGE = 2 * TK * ROWB;            // K tile + V tile
    static constexpr int STAGES = TK >= 128 ? 2 : (TK == 64 ? (WAVES == 8 ? 3 : 4) : 4);
    static constexpr int NI = TK / (2 * WAVES);            // DMA instructions per wave per tile
    static constexpr int XROW = 128 + 4;                   // padded fp32 row in the exchange area
    static constexpr int XSLOTS = (KS - 1) * R * NB;       // exchanged (wave, block) slots
    static constexpr int XBYTES = XSLOTS * 16 * (XROW + 2) * 4;
    static constexpr int LOOP_BYTES = STAGES * STAGE;
    static constexpr int IDX_BYTES = kGatherChunkMax * 4;
    static int constexpr maxi(int a, int b) { return a > b ? a : b; }
    static constexpr int SMEM_VERIFY = maxi(LOOP_BYTES, XBYTES);
    static constexpr int SMEM_GATHER = maxi(LOOP_BYTES + IDX_BYTES, XBYTES);
};

template <int WAVES, int R, int NB, bool GATHER>
__global__ __launch_bounds__(WAVES * 64, 1) void split_mfma(const SplitArgs a) {
    using S = MfmaShape<WAVES, R, NB>;
    constexpr int KS = S::KS, TK = S::TK, STAGES = S::STAGES, NI = S::NI;
    static_assert(NI >= 1 && (TK / 2) % WAVES == 0, "tile / wave split");
    constexpr int SMEM = GATHER ? S::SMEM_GATHER : S::SMEM_VERIFY;
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a scalar, so per-wave conditions compile to scalar branches
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = w / KS;   // query-row group of this wave
    const int ks = w % KS;   // 32-key sub-tile of this wave
    const int li = lane & 15;
    const int lj = lane >> 4;
    const int split = blockIdx.x;
    const int g = blockIdx.y;

    const int nblk = (a.M + 15) >> 4;
    const int nb_act = rg < nblk ? (nblk - rg + R - 1) / R : 0;

    const int64_t c0 = (int64_t)split * a.chunk_keys;
    const int64_t c1 = c0 + a.chunk_keys < a.n_keys ? c0 + a.chunk_keys : a.n_keys;
    const int n_pre_tiles = c1 > c0 ? (int)((c1 - c0 + TK - 1) / TK) : 0;
    const int n_tail_tiles = split == a.n_splits - 1 ? (a.T + TK - 1) / TK : 0;
    const int n_tiles = n_pre_tiles + n_tail_tiles;

    const char* kbase = (const char*)a.k + (size_t)g * (size_t)a.kv_head_stride * 2;
    const char* vbase = (const char*)a.v + (size_t)g * (size_t)a.kv_head_stride * 2;

    int32_t* idx_lds = (int32_t*)(smem + S::LOOP_BYTES);
    if constexpr (GATHER) {
        const int n = (int)(c1 > c0 ? c1 - c0 : 0);
        for (int i = tid; i < n; i += WAVES * 64) idx_lds[i] = a.idx[c0 + i];
        __syncthreads();
    }

    // Q^T as the B operand: lane (li, lj) holds query row li of the block,
    // head-dim elements 32*s + 8*lj .. +7.  Loads are unconditional (rows past
    // M read row 0 and are zeroed) and drained before the K/V pipeline starts,
    // so no wait for them is ever needed inside the tile loop.
    bf16x8 qop[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int r = (rg + b * R) * 16 + li;
        const bool ok = b < nb_act && r < a.M;
        const int t = ok ? r / a.G : 0;
        const int h = ok ? g * a.G + r % a.G : 0;
        const bf16x8* src = (const bf16x8*)((const __bf16*)a.q + ((size_t)t * a.Hq + h) * 128 + 8 * lj);
#pragma unroll
        for (int s = 0; s < 4; ++s) qop[b][s] = src[4 * s];
        if (!ok) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) qop[b][s][e] = (__bf16)0.0f;
        }
    }
    wait_vmcnt<0>();

    // One tile = TK K rows then TK V rows; each DMA instruction moves four
    // 256-byte rows (64 lanes x 16 bytes) into consecutive LDS.  Rows past the
    // end of the slice re-read a valid row; their scores are masked to -inf,
    // so they contribute exactly zero.
    auto issue_tile = [&](int tt, int st) {
        char* sbase = smem + st * S::STAGE;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int u = w * NI + i;
            const bool isv = u >= TK / 4;
            const int grp = isv ? u - TK / 4 : u;
            const int row = grp * 4 + lj;
            int64_t pos;
            if (tt < n_pre_tiles) {
                int64_t kk = c0 + (int64_t)tt * TK + row;
                if (kk >= c1) kk = c0;
                pos = GATHER ? (int64_t)idx_lds[kk - c0] : kk;
            } else {
                int jj = (tt - n_pre_tiles) * TK + row;
                if (jj >= a.T) jj = a.T - 1;
                pos = a.n_prefix + jj;
            }
            const char* src = (isv ? vbase : kbase) + pos * S::ROWB + 16 * (li ^ swz(row));
            char* dst = sbase + (isv ? TK * S::ROWB : 0) + grp * 1024;
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst,
                                             16, 0, 0);
        }
    };

    float m_run[NB], l_run[NB];
    f32x4 o[NB][8];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        m_run[b] = -INFINITY;
        l_run[b] = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[b][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < n_tiles) issue_tile(s, s);

    const float c = a.scale_log2;

    for (int tt = 0; tt < n_tiles; ++tt) {
        // Wait until this wave's loads of tile tt have landed; newer tiles
        // may stay in flight.
        const int newer = n_tiles - 1 - tt < STAGES - 2 ? n_tiles - 1 - tt : STAGES - 2;
        if constexpr (STAGES >= 4) {
            if (newer >= 2) wait_vmcnt<2 * NI>();
            else if (newer == 1) wait_vmcnt<NI>();
            else wait_vmcnt<0>();
        } else if constexpr (STAGES == 3) {
            if (newer >= 1) wait_vmcnt<NI>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        barrier_lds();
        if (tt + STAGES - 1 < n_tiles) issue_tile(tt + STAGES - 1, (tt + STAGES - 1) % STAGES);

        const char* Ks = smem + (tt % STAGES) * S::STAGE;
        const char* Vs = Ks + TK * S::ROWB;
        const bool tail = tt >= n_pre_tiles;
        const int64_t kstart = tail ? (int64_t)(tt - n_pre_tiles) * TK : c0 + (int64_t)tt * TK;
        const int64_t kend = tail ? a.T : c1;
        const bool full = !tail && kstart + TK <= kend;

        // S^T block (16 keys x 16 queries) per key half kb and query block b.
        f32x4 sc[2][NB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int b = 0; b < NB; ++b) sc[kb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = ks * 32 + kb * 16 + li;
                const bf16x8 kop = *(const bf16x8*)(Ks + row * S::ROWB + 16 * ((4 * s + lj) ^ swz(row)));
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < nb_act) sc[kb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[b][s], sc[kb][b], 0, 0, 0);
            }
        }

        // Mask keys past the slice end, and tree rows that are not ancestors.
        if (!full) {
            uint64_t nmask[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int r = (rg + b * R) * 16 + li;
                nmask[b] = (tail && r < a.M) ? a.mask[r / a.G] : ~0ull;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t key = kstart + ks * 32 + kb * 16 + 4 * lj + i;
                    const bool in_range = key < kend;
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        bool ok = in_range;
                        if (tail) ok = ok && ((nmask[b] >> (key & 63)) & 1ull);
                        if (!ok) sc[kb][b][i] = -INFINITY;
                    }
                }
        }

        // Online softmax per query row (one row per lane and block).
        bf16x8 pb[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b >= nb_act) continue;
            float mx = fmaxf(fmaxf(fmaxf(sc[0][b][0], sc[0][b][1]), fmaxf(sc[0][b][2], sc[0][b][3])),
                             fmaxf(fmaxf(sc[1][b][0], sc[1][b][1]), fmaxf(sc[1][b][2], sc[1][b][3])));
            mx = xor_max(mx, 16);
            mx = xor_max(mx, 32);
            const float mt = mx * c;
            const bool need = mt > m_run[b] + kRescaleTau;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mnew = need ? mt : m_run[b];
                const float alpha = mnew == m_run[b] ? 1.0f : exp2_fast(m_run[b] - mnew);
                l_run[b] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db) o[b][db] *= alpha;
                m_run[b] = mnew;
            }
            const float mu = m_run[b] == -INFINITY ? 0.0f : m_run[b];
            // p is rounded to bf16 for the PV product; the row sum adds the
            // same rounded values (v_dot2c_f32_bf16 with (1, 1)), so the
            // normalisation matches the weights actually applied to V.
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            float lsum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const bf16x2 pp = {(__bf16)exp2_fast(fmaf(sc[kb][b][i], c, -mu)),
                                       (__bf16)exp2_fast(fmaf(sc[kb][b][i + 1], c, -mu))};
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
                    pb[b][kb * 4 + i] = pp[0];
                    pb[b][kb * 4 + i + 1] = pp[1];
                }
            l_run[b] += lsum;
        }

        // O^T (d x queries) += V^T (d x keys) P^T (keys x queries).  The
        // transposed reads give lane (li, lj) V[key][16*db + li] for keys
        // 4*lj .. 4*lj+3 of each key half, matching P^T's layout.
        const int trow0 = ks * 32 + 4 * lj + (li >> 2);
        const int trow1 = trow0 + 16;
        const int tsel = (li >> 1) & 1;
        const char* vrow0 = Vs + trow0 * S::ROWB + 8 * (li & 1);
        const char* vrow1 = Vs + trow1 * S::ROWB + 8 * (li & 1);
        const int sw0 = swz(trow0) ^ tsel;
        const int sw1 = swz(trow1) ^ tsel;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vrow0 + 16 * ((2 * db) ^ sw0)));
            const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vrow1 + 16 * ((2 * db) ^ sw1)));
            const bf16x8 vop = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < nb_act) o[b][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[b], o[b][db], 0, 0, 0);
        }
    }

    // Row sums: each lane summed its own keys; add the four lane groups.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        l_run[b] = xor_sum(l_run[b], 16);
        l_run[b] = xor_sum(l_run[b], 32);
    }

    // Combine the KS key sub-tiles of each row group through LDS.
    float* xo = (float*)smem;
    float* xml = xo + S::XSLOTS * 16 * S::XROW;
    if constexpr (KS > 1) {
        barrier_lds();
        if (ks > 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b >= nb_act) continue;
                const int slot = ((ks - 1) * R + rg) * NB + b;
                float* dst = xo + (slot * 16 + li) * S::XROW + 4 * lj;
#pragma unroll
                for (int db = 0; db < 8; ++db) *(f32x4*)(dst + 16 * db) = o[b][db];
                if (lj == 0) {
                    xml[slot * 32 + li] = m_run[b];
                    xml[slot * 32 + 16 + li] = l_run[b];
                }
            }
        }
        barrier_lds();
        if (ks > 0) return;
    }

#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (b >= nb_act) continue;
        const int r = (rg + b * R) * 16 + li;
        float mk[KS], wk[KS];
        mk[0] = m_run[b];
        float mmax = m_run[b];
#pragma unroll
        for (int k2 = 1; k2 < KS; ++k2) {
            const int slot = ((k2 - 1) * R + rg) * NB + b;
            mk[k2] = xml[slot * 32 + li];
            mmax = fmaxf(mmax, mk[k2]);
        }
        float L = 0.0f;
#pragma unroll
        for (int k2 = 0; k2 < KS; ++k2) {
            wk[k2] = mk[k2] == -INFINITY ? 0.0f : exp2_fast(mk[k2] - mmax);
            const float lk = k2 == 0 ? l_run[b] : xml[(((k2 - 1) * R + rg) * NB + b) * 32 + 16 + li];
            L += wk[k2] * lk;
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        if (r >= a.M) continue;
        const int t = r / a.G;
        const int h = g * a.G + r % a.G;
        const size_t orow = ((size_t)split * a.T + t) * a.Hq + h;
        float* dst = a.part_o + orow * 128 + 4 * lj;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            f32x4 acc = o[b][db] * wk[0];
#pragma unroll
            for (int k2 = 1; k2 < KS; ++k2) {
                const int slot = ((k2 - 1) * R + rg) * NB + b;
                acc += wk[k2] * *(const f32x4*)(xo + (slot * 16 + li) * S::XROW + 16 * db + 4 * lj);
            }
            *(f32x4*)(dst + 16 * db) = acc * inv;
        }
        if (lj == 0) a.part_lse[orow] = L > 0.0f ? (mmax + __log2f(L)) * kLn2 : -INFINITY;
    }
}

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
// One wavefront per output row: lanes hold the split LSEs (64 at a time),
// wave reductions give the row's LSE, and each lane accumulates d/64
// consecutive columns over the splits with coalesced loads.
template <int D>
__global__ __launch_bounds__(256) void lse_merge(int n_splits, int64_t n_rows,
                                                 const float* __restrict__ part_o,
                                                 const float* __restrict__ part_lse,
                                                 float* __restrict__ o, float* __restrict__ lse) {
    constexpr int PER = D / 64;
    constexpr float kLog2e = 1.44269504088896340736f;
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;
    float mx = -INFINITY;
    for (int s0 = 0; s0 < n_splits; s0 += 64)
        if (s0 + lane < n_splits) mx = fmaxf(mx, part_lse[(int64_t)(s0 + lane) * n_rows + r]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = xor_max(mx, m);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    if (mx == -INFINITY) {
#pragma unroll
        for (int e = 0; e < PER; ++e) o[r * D + lane * PER + e] = 0.0f;
        if (lane == 0) lse[r] = -INFINITY;
        return;
    }
    float sum = 0.0f;
    for (int s0 = 0; s0 < n_splits; s0 += 64)
        if (s0 + lane < n_splits) {
            const float ls = part_lse[(int64_t)(s0 + lane) * n_rows + r];
            sum += ls == -INFINITY ? 0.0f : exp2f((ls - mx) * kLog2e);
        }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum = xor_sum(sum, m);
    const float L = mx + logf(sum);
    for (int s0 = 0; s0 < n_splits; s0 += 64) {
        float wl = 0.0f;
        if (s0 + lane < n_splits) {
            const float ls = part_lse[(int64_t)(s0 + lane) * n_rows + r];
            wl = ls == -INFINITY ? 0.0f : exp2f((ls - L) * kLog2e);
        }
        const int n = n_splits - s0 < 64 ? n_splits - s0 : 64;
#pragma unroll 8
        for (int j = 0; j < n; ++j) {
            const float wj = __shfl(wl, j);
            const float* src = part_o + ((int64_t)(s0 + j) * n_rows + r) * D + lane * PER;
            if constexpr (PER == 2) {
                const float2 x = *(const float2*)src;
                acc[0] = fmaf(wj, x.x, acc[0]);
                acc[1] = fmaf(wj, x.y, acc[1]);
            } else {
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, src[e], acc[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) o[r * D + lane * PER + e] = acc[e];
    if (lane == 0) lse[r] = L;
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
bool mfma_config_for(int M, MfmaConfig* cfg) {
    // At most 3 query blocks per wave with two waves per SIMD (256 registers
    // each); the 4-block shape runs one wave per SIMD.
    const int nblk = (M + 15) / 16;
    if (nblk <= 2) *cfg = {4, 1, 2};
    else if (nblk <= 4) *cfg = {8, 2, 2};
    else if (nblk <= 8) *cfg = {8, 4, 2};
    else if (nblk <= 12) *cfg = {8, 4, 3};
    else if (nblk <= 16) *cfg = {4, 4, 4};
    else return false;
    return true;
}

template <int W, int R, int NB>
static hipError_t launch_mfma_t(bool gather, const SplitArgs& a, int n_kv_heads, hipStream_t stream) {
    const dim3 grid(a.n_splits, n_kv_heads);
    if (gather) hipLaunchKernelGGL((split_mfma<W, R, NB, true>), grid, dim3(W * 64), 0, stream, a);
    else hipLaunchKernelGGL((split_mfma<W, R, NB, false>), grid, dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_split_mfma(const MfmaConfig& cfg, bool gather, const SplitArgs& a, int n_kv_heads,
                             hipStream_t stream) {
    if (cfg.waves == 4 && cfg.rgroups == 1 && cfg.nb == 2) return launch_mfma_t<4, 1, 2>(gather, a, n_kv_heads, stream);
    if (cfg.waves == 8 && cfg.rgroups == 2 && cfg.nb == 2) return launch_mfma_t<8, 2, 2>(gather, a, n_kv_heads, stream);
    if (cfg.waves == 8 && cfg.rgroups == 4 && cfg.nb == 2) return launch_mfma_t<8, 4, 2>(gather, a, n_kv_heads, stream);
    if (cfg.waves == 8 && cfg.rgroups == 4 && cfg.nb == 3) return launch_mfma_t<8, 4, 3>(gather, a, n_kv_heads, stream);
    if (cfg.waves == 4 && cfg.rgroups == 4 && cfg.nb == 4) return launch_mfma_t<4, 4, 4>(gather, a, n_kv_heads, stream);
    return hipErrorInvalidValue;
}

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

hipError_t launch_lse_merge(int n_splits, int64_t n_rows, int d, const float* part_o,
                            const float* part_lse, float* o, float* lse, hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    if (d == 128 || d == 64) {
        const dim3 grid((unsigned)((n_rows + 3) / 4));
        if (d == 128)
            hipLaunchKernelGGL(lse_merge<128>, grid, dim3(256), 0, stream, n_splits, n_rows, part_o, part_lse, o, lse);
        else
            hipLaunchKernelGGL(lse_merge<64>, grid, dim3(256), 0, stream, n_splits, n_rows, part_o, part_lse, o, lse);
        return hipGetLastError();
    }
    const int64_t n = n_rows * d;
    const dim3 grid((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(lse_merge_generic, grid, dim3(256), 0, stream, n_splits, n_rows, d, part_o, part_lse, o, lse);
    return hipGetLastError();
}

}  // namespace tsw
