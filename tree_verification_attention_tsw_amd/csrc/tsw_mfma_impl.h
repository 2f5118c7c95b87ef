// Matrix-core split kernel for tree-verification attention (gfx950, bf16,
// head dim 128) -- template code, instantiated once per shape by
// tsw_mfma_inst.hip.
//
// One work-group per (split, kv head): it streams a contiguous slice of that
// head's key list once (prefix keys, then -- in the last split -- the tree's
// own rows under the ancestor mask) and applies it to all M = T * (Hq/Hkv)
// query rows that share the head, so every K/V byte leaves HBM once per call
// (the GQA head group and all tree nodes ride on one K/V stream).  Sources:
// "TokenSwift - A framework for accelerating the generation of ultra-long
// text" (aiboss88 project page), technical principles, tree-based
// multi-candidate verification; Tencent Cloud article "90分钟生成10万Token，
// 新框架实现3倍无损加速超长文本生成", 技术原理 figure text (verification with
// the full KV cache) and 无损的输出质量 (draft pass = same model over a
// partial KV cache).
//
// Layout of the work: four wavefronts (one per SIMD, up to 512 registers) or
// eight (two per SIMD, 256 registers), each owning NB or NB-1 blocks of 16
// query rows (R row groups) and one 32-key sub-tile of every key tile
// (W/R sub-tiles per tile).  Per tile:
//   * K and V rows move HBM -> LDS with LDS-DMA loads (buffer loads over the
//     split's rows of a contiguous cache and over one page's rows for whole
//     paged prefix tiles, global loads for gathered rows and the other paged
//     tiles; streaming cache policy; K and V rows each with their own chunk
//     swizzle) into a 128 KB ring of two 128-key load groups: one group
//     is in flight while the other is computed on, and one work-group
//     barrier per group recycles its stages.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with key rows on the M axis and
//     query rows on N, so every lane owns one query row of each block.
//   * O += P V on the same instruction (queries on rows); V operands come
//     straight from row-major LDS through ds_read_b64_tr_b16.
//   * Four-wave shapes pipeline blocks (the Q K products of block b+1 share
//     a basic block with the exponentials of block b); eight-wave shapes run
//     Q K of all blocks, the exponentials, then P V, and leave the overlap to
//     the SIMD's other wave.
//
// Softmax without a running maximum.  The fast pass exponentiates scores
// directly, p = 2^(s * scale * log2 e), and accumulates O and l = sum p.
// That is the exact softmax as long as every row's logits stay within about
// [-41, +88] nats (no overflow of p, l or O; the largest p not vanishing).
// A row outside that range shows up at the end as a non-finite or vanishing
// sum; its work-group then reruns the split exactly: one pass for the row
// maxima, one pass with p = 2^(s*c - max) <= 1.  The hot loop therefore
// carries no per-tile maximum, rescale or cross-lane reduction.
#pragma once

#include <type_traits>

#include "tsw_device.h"
#include "tsw_internal.h"


namespace tsw {
namespace mfma {

// Fast-pass acceptance: row sums below this mean the largest p was tiny
// (logits far below zero) and precision could suffer; rerun exactly.
constexpr float kMinRowSum = 0x1p-60f;

template <int W_, int R_, int NB_, int MODE_>
struct Shape {
    static constexpr int R = R_;
    static constexpr int NB = NB_;
    static constexpr int WAVES = W_;
    static constexpr int KS = WAVES / R;            // 32-key sub-tiles per tile
    static constexpr int TK = 32 * KS;              // keys per tile
    static constexpr int ROWB = 256;                // bytes per K or V row
    static constexpr int STAGE = 2 * TK * ROWB;     // one K tile + one V tile
    static constexpr int NI = TK / (2 * WAVES);     // DMA instructions per wave per tile
    // LDS beyond the ring: the work-group vote, the tree mask, and for the
    // gather and paged variants the staged index or page-table slice.
    static constexpr int POOL = WAVES * 4;            // the work-group vote
    static constexpr int MASK_BYTES = 64 * 8;
    // (paged draft pass: the slice's pool rows, then the tree rows' after it)
    static constexpr int IDX_BYTES = MODE_ == kModeContig ? 0
                                     : MODE_ == kModePagedGather ? (kGatherChunkMax + 64) * 4
                                                                 : kGatherChunkMax * 4;
    static constexpr int RESERVE = ((POOL + MASK_BYTES + 255) & ~255) + IDX_BYTES;
    // Loads are issued, waited for and recycled in groups of GT tiles, 128
    // keys (32 KB of K and 32 KB of V) per group, with one barrier per group.
    // The ring holds two groups, one in flight while the other is computed
    // on; on MI355X that streams faster than more, smaller stages in the
    // same LDS.
    static constexpr int GT = TK >= 128 ? 1 : 128 / TK;
    static constexpr int STAGES_FIT = (160 * 1024 - RESERVE) / STAGE;
    static constexpr int STAGES = 2 * GT;
    static constexpr int RING = STAGES * STAGE;
    // Epilogue exchange: each wave parks, per block, the column blocks the
    // other KS-1 waves of its row group finish (one f32x4 per lane each),
    // plus its per-row (m, l).
    static constexpr int DPW = 8 / KS;                 // column blocks finished per wave
    static constexpr int XSLOTS = (KS - 1) * R * NB;   // parked blocks' worth of columns
    static constexpr int XO_BYTES = XSLOTS * 8 * 64 * 16;
    static constexpr int XBYTES = XO_BYTES + R * NB * KS * 32 * 4;
    // ring (+ index slice) during the loop, the KS exchange afterwards
    static constexpr int LOOP_BYTES = RING + IDX_BYTES;
    static constexpr int SMEM = LOOP_BYTES > XBYTES ? LOOP_BYTES : XBYTES;
    static_assert(STAGES <= STAGES_FIT, "two load groups fit the LDS");
    static_assert(GT * NI < 64, "vmcnt range");
    static_assert((TK / 4) % NI == 0, "a wave's loads are all K rows or all V rows");
};

struct Ctx {
    char* smem;
    const int32_t* idx_lds;      // gather: index slice; paged: page-table slices;
                                 // paged gather: pool rows of the slice and the tree rows
    const uint64_t* mask_lds;    // the tree mask, copied to LDS
    const char* kbase;           // this kv head's cache (paged: the page pool)
    const char* vbase;
    const __bf16* q;             // this sequence's queries
    int64_t n_prefix;            // this sequence's committed length
    int64_t c0, c1;      // prefix key range [c0, c1) of this split
    int64_t pg0, tpg0;   // paged: first page of the slice and of the tree rows
    const char* kseg;    // contiguous: the split's first K and V rows, and the
    const char* vseg;    // bytes from there it reads (its slice, plus the
    uint32_t seg_bytes;  // tree rows in the last split)
    int64_t row0;        // partial-output row of (split, sequence, node 0)
    int npg;             // paged: pages staged for the slice
    int n_pre_tiles, n_tiles;
    int lane, li, lj, w, rg, ks, split, g;
};

// Issue the DMA loads of tile tt into ring stage st.  One instruction moves
// four 256-byte rows (64 lanes x 16 bytes) into consecutive LDS; lane (li,
// lj) of instruction i writes logical chunk li ^ swz(row) (V) or li ^ swz_k(row)
// (K) of its row.  Rows
// past the slice end re-read a valid row (their scores are masked to -inf).
template <class S, int MODE>
__device__ __forceinline__ void issue_tile(const SplitArgs& a, const Ctx& cx, int tt, int st) {
    char* sbase = cx.smem + st * S::STAGE;
    // waves 0 .. W/2-1 load K rows, the others V rows (uniform per wave);
    // their LDS rows have different swizzles
    const bool wave_v = cx.w * S::NI >= S::TK / 4;
    const int v_bits = wave_v ? 15 : 0;
    auto row_swz = [&](int row) { return swz_k(row) ^ ((swz(row) ^ swz_k(row)) & v_bits); };
    const bool pre = tt < cx.n_pre_tiles;
    const int64_t k0 = cx.c0 + (int64_t)tt * S::TK;
    if constexpr (MODE == kModeContig) {
        // Consecutive cache rows, prefix and tree tiles alike: buffer loads
        // over the split's rows, a scalar offset per tile (its first row)
        // and a fixed 32-bit offset per lane and instruction, so a load costs
        // no vector instruction.  Rows past the split's range (the ragged
        // end of the slice, the tree tile's padding) read as zeros; their
        // scores are masked to -inf.
        const __amdgpu_buffer_rsrc_t krs = raw_rsrc(cx.kseg, cx.seg_bytes);
        const __amdgpu_buffer_rsrc_t vrs = raw_rsrc(cx.vseg, cx.seg_bytes);
        const uint32_t r0 = pre ? (uint32_t)tt * S::TK
                                : (uint32_t)(cx.n_prefix - cx.c0) + (uint32_t)(tt - cx.n_pre_tiles) * S::TK;
#pragma unroll
        for (int i = 0; i < S::NI; ++i) {
            const int u = cx.w * S::NI + i;
            const bool isv = wave_v;
            const int grp = isv ? u - S::TK / 4 : u;
            const int row = grp * 4 + cx.lj;
            const uint32_t off = (uint32_t)(row * S::ROWB + 16 * (cx.li ^ (isv ? swz(row) : swz_k(row))));
            char* dst = sbase + (isv ? S::TK * S::ROWB : 0) + grp * 1024;
            buffer_load_lds16(isv ? vrs : krs, dst, off, r0 * (uint32_t)S::ROWB);
        }
        return;
    }
    if constexpr (MODE == kModePagedGather) {
        // paged draft pass: the staged entries are pool rows (page number
        // times page_rows plus the row in the page), prefix slice first and
        // the tree rows at kGatherChunkMax
#pragma unroll
        for (int i = 0; i < S::NI; ++i) {
            const int u = cx.w * S::NI + i;
            const bool isv = wave_v;
            const int grp = isv ? u - S::TK / 4 : u;
            const int row = grp * 4 + cx.lj;
            int slot;
            if (pre) {
                int64_t kk = k0 + row;
                if (kk >= cx.c1) kk = cx.c0;
                slot = (int)(kk - cx.c0);
            } else {
                int jj = (tt - cx.n_pre_tiles) * S::TK + row;
                if (jj >= a.T) jj = a.T - 1;
                slot = kGatherChunkMax + jj;
            }
            const uint32_t prow = (uint32_t)cx.idx_lds[slot];
            const char* src = (isv ? cx.vbase : cx.kbase) + (uint64_t)(prow >> a.page_shift) * (uint64_t)a.page_bytes +
                              (uint32_t)((prow & (uint32_t)(a.page_rows - 1)) * S::ROWB +
                                         16 * (cx.li ^ (isv ? swz(row) : swz_k(row))));
            char* dst = sbase + (isv ? S::TK * S::ROWB : 0) + grp * 1024;
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0,
                                             kStreamAux);
        }
    } else if constexpr (MODE != kModePaged) {
#pragma unroll
        for (int i = 0; i < S::NI; ++i) {
            const int u = cx.w * S::NI + i;
            const bool isv = wave_v;
            const int grp = isv ? u - S::TK / 4 : u;
            const int row = grp * 4 + cx.lj;
            int64_t pos;
            if (pre) {
                int64_t kk = k0 + row;
                if (kk >= cx.c1) kk = cx.c0;
                pos = MODE == kModeGather ? (int64_t)cx.idx_lds[kk - cx.c0] : kk;
            } else {
                int jj = (tt - cx.n_pre_tiles) * S::TK + row;
                if (jj >= a.T) jj = a.T - 1;
                pos = cx.n_prefix + jj;
            }
            const char* src = (isv ? cx.vbase : cx.kbase) + pos * S::ROWB +
                              16 * (cx.li ^ (isv ? swz(row) : swz_k(row)));
            char* dst = sbase + (isv ? S::TK * S::ROWB : 0) + grp * 1024;
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0,
                                             kStreamAux);
        }
    } else {
        if (pre && k0 + S::TK <= cx.c1) {
            // A whole prefix tile: an instruction's four rows start at a
            // multiple of four, so they share a page (pages hold at least 16
            // rows).  Its page number is read once (a uniform LDS read) and
            // the load goes through a buffer over this head's rows of that
            // page: a scalar base and row offset per instruction, a fixed
            // 32-bit offset per lane, no vector address arithmetic.
            uint32_t page[S::NI];
#pragma unroll
            for (int i = 0; i < S::NI; ++i) {
                const int u = cx.w * S::NI + i;
                const int grp = u >= S::TK / 4 ? u - S::TK / 4 : u;
                page[i] = (uint32_t)cx.idx_lds[(int)(((k0 + grp * 4) >> a.page_shift) - cx.pg0)];
            }
            const uint32_t head_rows_bytes = (uint32_t)a.page_rows * S::ROWB;
#pragma unroll
            for (int i = 0; i < S::NI; ++i) {
                const int u = cx.w * S::NI + i;
                const bool isv = wave_v;
                const int grp = isv ? u - S::TK / 4 : u;
                const uint32_t pg = __builtin_amdgcn_readfirstlane(page[i]);
                const char* pbase = (isv ? cx.vbase : cx.kbase) + (uint64_t)pg * (uint64_t)a.page_bytes;
                const uint32_t r0 = (uint32_t)((k0 + grp * 4) & (a.page_rows - 1));
                const int row = grp * 4 + cx.lj;
                const uint32_t off =
                    (uint32_t)(cx.lj * S::ROWB + 16 * (cx.li ^ (isv ? swz(row) : swz_k(row))));
                char* dst = sbase + (isv ? S::TK * S::ROWB : 0) + grp * 1024;
                buffer_load_lds16(raw_rsrc(pbase, head_rows_bytes), dst, off, r0 * (uint32_t)S::ROWB);
            }
            return;
        }
        // paged, other tiles (the ragged end of a slice, the tree rows):
        // every load's page number is read from the staged table first, then
        // each address is one multiply-add on it
        int64_t pos[S::NI];
        uint32_t page[S::NI];
#pragma unroll
        for (int i = 0; i < S::NI; ++i) {
            const int u = cx.w * S::NI + i;
            const int grp = u >= S::TK / 4 ? u - S::TK / 4 : u;
            const int row = grp * 4 + cx.lj;
            if (pre) {
                int64_t kk = k0 + row;
                if (kk >= cx.c1) kk = cx.c0;
                pos[i] = kk;
            } else {
                int jj = (tt - cx.n_pre_tiles) * S::TK + row;
                if (jj >= a.T) jj = a.T - 1;
                pos[i] = cx.n_prefix + jj;
            }
            const int64_t lp = pos[i] >> a.page_shift;
            const int slot = pre ? (int)(lp - cx.pg0) : cx.npg + (int)(lp - cx.tpg0);
            page[i] = (uint32_t)cx.idx_lds[slot];
        }
#pragma unroll
        for (int i = 0; i < S::NI; ++i) {
            const int u = cx.w * S::NI + i;
            const bool isv = wave_v;
            const int grp = isv ? u - S::TK / 4 : u;
            const int row = grp * 4 + cx.lj;
            const char* src = (isv ? cx.vbase : cx.kbase) + (uint64_t)page[i] * (uint64_t)a.page_bytes +
                              (uint32_t)((pos[i] & (a.page_rows - 1)) * S::ROWB +
                                         16 * (cx.li ^ row_swz(row)));
            char* dst = sbase + (isv ? S::TK * S::ROWB : 0) + grp * 1024;
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0,
                                             kStreamAux);
        }
    }
}

// K operands of this wave's 32-key sub-tile: lane (li, lj) holds key row
// kb*16 + li, head-dim elements 32*s + 8*lj .. +7.  The tile's stage is Ks +
// SOFF; a constant SOFF lands in the reads' offset fields, so the tiles of a
// load group share their address arithmetic.
template <class S, int SOFF = 0>
__device__ __forceinline__ void load_k(const char* Ks, const Ctx& cx, bf16x8 (&kop)[2][4]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int row = cx.ks * 32 + kb * 16 + cx.li;
        const char* base = Ks + SOFF + row * S::ROWB;
        const int sw = swz_k(row);
#pragma unroll
        for (int s = 0; s < 4; ++s) kop[kb][s] = *(const bf16x8*)(base + 16 * ((4 * s + cx.lj) ^ sw));
    }
}

// V operands: the transposed reads give lane (li, lj) V[key][16*db + li] for
// keys 4*lj .. 4*lj+3 of each 16-key half, matching P's K-slot layout.
// Rows trow and trow + 16 share their swizzle (it depends on the low four
// row bits only), so the second half is the first at a constant offset.
// The V tile follows the K tile in the stage at Ks + SOFF.
template <class S, int SOFF = 0>
__device__ __forceinline__ void load_v(const char* Ks, const Ctx& cx, bf16x8 (&vop)[8]) {
    constexpr int VOFF = SOFF + S::TK * S::ROWB;
    const int trow0 = cx.ks * 32 + 4 * cx.lj + (cx.li >> 2);
    const int tsel = (cx.li >> 1) & 1;
    const char* vrow0 = Ks + trow0 * S::ROWB + 8 * (cx.li & 1);
    const int sw0 = swz(trow0) ^ tsel;
    bf16x4 v0[8], v1[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        v0[db] = ds_read_tr16_b64_at<VOFF>(vrow0 + 16 * ((2 * db) ^ sw0));
        v1[db] = ds_read_tr16_b64_at<VOFF + 16 * S::ROWB>(vrow0 + 16 * ((2 * db) ^ sw0));
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        lds_wait(v0[db], v1[db]);
        vop[db] = __builtin_shufflevector(v0[db], v1[db], 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// Starting values of a block's S^T accumulators.  Unmasked tiles start from
// zero; MASKED tiles (the ragged end of a slice, the tree's own rows) start
// from 0 / -inf, -inf for keys past the slice end and for tree rows that are
// not ancestors-or-self of the query's node, so the scores are never touched
// after the products.
template <class S, bool MASKED>
__device__ __forceinline__ void s_init(const SplitArgs& a, const Ctx& cx, int tt, int b, f32x4 (&s0)[2]) {
    if constexpr (!MASKED) {
        s0[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        s0[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        const bool tail = tt >= cx.n_pre_tiles;
        const int64_t kstart = tail ? (int64_t)(tt - cx.n_pre_tiles) * S::TK : cx.c0 + (int64_t)tt * S::TK;
        const int64_t kend = tail ? a.T : cx.c1;
        const int r = (cx.rg + b * S::R) * 16 + cx.li;
        const uint64_t nmask = (tail && r < a.M) ? cx.mask_lds[r / a.G] : ~0ull;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t key = kstart + cx.ks * 32 + kb * 16 + 4 * cx.lj + i;
                bool ok = key < kend;
                if (tail) ok = ok && ((nmask >> (key & 63)) & 1ull);
                s0[kb][i] = ok ? 0.0f : -INFINITY;
            }
    }
}

// S^T for one query block: 16 keys x 16 queries per key half.
__device__ __forceinline__ void qk_block(const bf16x8 (&kop)[2][4], const bf16x8 (&qb)[4], f32x4 (&sc)[2]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb][s], qb[s], sc[kb], 0, 0, 0);
}

// p = 2^(s*c - mu) for one block, rounded to bf16 for the P V product; the
// row sum adds the same rounded values (v_dot2c_f32_bf16 with (1, 1)), so
// the normalisation matches the weights actually applied to V.  With SPLIT
// (masked tiles: the ragged end of a slice and the tree's own rows, where a
// row may see only a handful of keys and single rounding errors do not
// average out) p is carried as bf16 pb + bf16 pl, pl the rounding residue,
// about 16 significant bits; both go through P V and into the row sum.
template <bool SHIFT, bool SPLIT = false>
__device__ __forceinline__ void softmax_block(const f32x4 (&sc)[2], float c, float mu, float& l, bf16x8& pb,
                                              bf16x8& pl) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            const float t0 = SHIFT ? fmaf(sc[kb][i], c, -mu) : sc[kb][i] * c;
            const float t1 = SHIFT ? fmaf(sc[kb][i + 1], c, -mu) : sc[kb][i + 1] * c;
            const float e0 = exp2_fast(t0), e1 = exp2_fast(t1);
            const bf16x2 pp = {(__bf16)e0, (__bf16)e1};
            l = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l, false);
            pb[kb * 4 + i] = pp[0];
            pb[kb * 4 + i + 1] = pp[1];
            if constexpr (SPLIT) {
                // e - hi is exact in float; -inf scores give e = 0, hi = 0
                const bf16x2 rr = {(__bf16)(e0 - (float)pp[0]), (__bf16)(e1 - (float)pp[1])};
                l = __builtin_amdgcn_fdot2_f32_bf16(rr, ones, l, false);
                pl[kb * 4 + i] = rr[0];
                pl[kb * 4 + i + 1] = rr[1];
            }
        }
}

template <bool SHIFT>
__device__ __forceinline__ void softmax_block(const f32x4 (&sc)[2], float c, float mu, float& l, bf16x8& pb) {
    bf16x8 unused;
    softmax_block<SHIFT, false>(sc, c, mu, l, pb, unused);
}

__device__ __forceinline__ void pv_block(const bf16x8& pb, const bf16x8 (&vop)[8], f32x4 (&ob)[8]) {
#pragma unroll
    for (int db = 0; db < 8; ++db) ob[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, vop[db], ob[db], 0, 0, 0);
}

// Root-row scores (node 0's query heads: rows r < G <= 16, all in block 0
// of row group 0), lane li holding row li and four consecutive keys per key
// half.  Prefix keys only; in a masked tile only those before the slice end.
template <class S, bool MASKED>
__device__ __forceinline__ void emit_root(const SplitArgs& a, const Ctx& cx, int tt, const f32x4 (&sc)[2]) {
    if (cx.rg != 0) return;                          // uniform
    if (MASKED && tt >= cx.n_pre_tiles) return;      // the tree's own rows
    if (cx.li >= a.G) return;
    float* dst = a.root_s + (size_t)(cx.g * a.G + cx.li) * a.root_stride +
                 (cx.c0 + (int64_t)tt * S::TK + cx.ks * 32 + 4 * cx.lj);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if constexpr (!MASKED) {
            *(f32x4*)(dst + kb * 16) = sc[kb];
        } else {
            const int64_t key = cx.c0 + (int64_t)tt * S::TK + cx.ks * 32 + kb * 16 + 4 * cx.lj;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key + i < cx.c1) dst[kb * 16 + i] = sc[kb][i];
        }
    }
}

// One key tile for a wave owning NBA query blocks: Q K of block b+1 is
// issued next to the exponentials of block b (independent), then P V of
// block b.  SHIFT subtracts the row maxima m (exact pass).
template <class S, int NBA, bool MASKED, bool SHIFT, bool EMIT>
__device__ __forceinline__ void tile_pv(const SplitArgs& a, const Ctx& cx, int tt, float c, const bf16x8 (&kop)[2][4],
                                        const bf16x8 (&vop)[8], const bf16x8 (&qop)[NBA][4], const float (&m)[NBA],
                                        float (&l)[NBA], f32x4 (&o)[NBA][8]) {
    f32x4 sc[2][2];
    s_init<S, MASKED>(a, cx, tt, 0, sc[0]);
    qk_block(kop, qop[0], sc[0]);
#pragma unroll
    for (int b = 0; b < NBA; ++b) {
        if (b + 1 < NBA) {
            s_init<S, MASKED>(a, cx, tt, b + 1, sc[(b + 1) & 1]);
            qk_block(kop, qop[b + 1], sc[(b + 1) & 1]);
        }
        if constexpr (EMIT)
            if (b == 0) emit_root<S, MASKED>(a, cx, tt, sc[0]);
        bf16x8 pb, pl;
        // a wave whose key sub-tiles held no visible key for a row has m = -inf
        softmax_block<SHIFT, MASKED>(sc[b & 1], c, (SHIFT && m[b] != -INFINITY) ? m[b] : 0.0f, l[b], pb, pl);
        pv_block(pb, vop, o[b]);
        if constexpr (MASKED) pv_block(pl, vop, o[b]);
    }
}

// The same tile for waves that share their SIMD with a second wave (256
// registers each): Q K for all blocks one head-dim step at a time, the
// exponentials of all blocks, then P V one V column block at a time, so only
// a step's K operands and one V operand are live.  The other wave on the
// SIMD fills the matrix pipe while this one exponentiates.
template <class S, int NBA, bool MASKED, bool SHIFT, bool EMIT, int SOFF = 0>
__device__ __forceinline__ void tile_pv_shared(const SplitArgs& a, const Ctx& cx, int tt, float c, const char* Ks,
                                               const bf16x8 (&qop)[NBA][4], const float (&m)[NBA],
                                               float (&l)[NBA], f32x4 (&o)[NBA][8]) {
    constexpr int VOFF = SOFF + S::TK * S::ROWB;
    const int trow0 = cx.ks * 32 + 4 * cx.lj + (cx.li >> 2);
    const int tsel = (cx.li >> 1) & 1;
    const char* vrow0 = Ks + trow0 * S::ROWB + 8 * (cx.li & 1);
    const int sw0 = swz(trow0) ^ tsel;
    f32x4 sc[NBA][2];
#pragma unroll
    for (int b = 0; b < NBA; ++b) s_init<S, MASKED>(a, cx, tt, b, sc[b]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int row = cx.ks * 32 + kb * 16 + cx.li;
        const char* base = Ks + SOFF + row * S::ROWB;
        const int sw = swz_k(row);
        if constexpr (S::NB <= 2) {
            // the four head-dim chunks of this 16-key half are read before
            // their products, so each product waits only for its own chunk
            // (GQA-14B's 13 blocks on (8,8,2): 107.1 -> 104.1 us per split
            // kernel; the three-block shapes read one chunk at a time: the
            // deeper reads cost them registers and gained nothing)
            bf16x8 kq[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) kq[s] = *(const bf16x8*)(base + 16 * ((4 * s + cx.lj) ^ sw));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int b = 0; b < NBA; ++b)
                    sc[b][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq[s], qop[b][s], sc[b][kb], 0, 0, 0);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 kop = *(const bf16x8*)(base + 16 * ((4 * s + cx.lj) ^ sw));
#pragma unroll
                for (int b = 0; b < NBA; ++b)
                    sc[b][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[b][s], sc[b][kb], 0, 0, 0);
            }
        }
    }
    if constexpr (EMIT) emit_root<S, MASKED>(a, cx, tt, sc[0]);
    // V rows are addressed from the K stage (vrow0, VOFF above): the stage
    // offset, the V tile and the second 16-row half (same swizzle) are
    // constant offsets of the read.
    // V operands go through a window of VW column blocks (two transposed
    // reads each).  The first VW blocks are read before the exponentials, so
    // their latency hides under them; each later block is read as the window
    // moves, and block db waits only for its own two reads.  Deeper windows
    // push the three-block waves of the larger shapes into register spills,
    // so those keep a window of one block read after the exponentials.
    constexpr int VW = NBA >= 3 ? (S::R == 8 ? 1 : 2) : 4;
    if constexpr (MASKED) {
        // Masked tiles (at most two per split: the ragged end of a slice and
        // the tree's own rows): a row here may see only a handful of keys,
        // whose rounding errors would not average out, so P travels as two
        // bf16 parts; V column blocks are read one at a time after the
        // exponentials, which keeps the extra parts within the registers.
        bf16x8 pb[NBA], pl[NBA];
#pragma unroll
        for (int b = 0; b < NBA; ++b)
            softmax_block<SHIFT, true>(sc[b], c, (SHIFT && m[b] != -INFINITY) ? m[b] : 0.0f, l[b], pb[b], pl[b]);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            bf16x4 c0 = ds_read_tr16_b64_at<VOFF>(vrow0 + 16 * ((2 * db) ^ sw0));
            bf16x4 c1 = ds_read_tr16_b64_at<VOFF + 16 * S::ROWB>(vrow0 + 16 * ((2 * db) ^ sw0));
            lds_wait(c0, c1);
            const bf16x8 vop = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int b = 0; b < NBA; ++b) {
                o[b][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[b], vop, o[b][db], 0, 0, 0);
                o[b][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[b], vop, o[b][db], 0, 0, 0);
            }
        }
        return;
    }
    if constexpr (VW == 1) {
        bf16x8 pb[NBA];
#pragma unroll
        for (int b = 0; b < NBA; ++b)
            softmax_block<SHIFT>(sc[b], c, (SHIFT && m[b] != -INFINITY) ? m[b] : 0.0f, l[b], pb[b]);
        bf16x4 c0 = ds_read_tr16_b64_at<VOFF>(vrow0 + 16 * (0 ^ sw0));
        bf16x4 c1 = ds_read_tr16_b64_at<VOFF + 16 * S::ROWB>(vrow0 + 16 * (0 ^ sw0));
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            lds_wait(c0, c1);
            const bf16x8 vop = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
            if (db + 1 < 8) {
                c0 = ds_read_tr16_b64_at<VOFF>(vrow0 + 16 * ((2 * (db + 1)) ^ sw0));
                c1 = ds_read_tr16_b64_at<VOFF + 16 * S::ROWB>(vrow0 + 16 * ((2 * (db + 1)) ^ sw0));
            }
#pragma unroll
            for (int b = 0; b < NBA; ++b)
                o[b][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[b], vop, o[b][db], 0, 0, 0);
        }
        return;
    }
    bf16x4 va[8], vb[8];
#pragma unroll
    for (int db = 0; db < VW; ++db) {
        va[db] = ds_read_tr16_b64_at<VOFF>(vrow0 + 16 * ((2 * db) ^ sw0));
        vb[db] = ds_read_tr16_b64_at<VOFF + 16 * S::ROWB>(vrow0 + 16 * ((2 * db) ^ sw0));
    }
    bf16x8 pb[NBA];
#pragma unroll
    for (int b = 0; b < NBA; ++b)
        softmax_block<SHIFT>(sc[b], c, (SHIFT && m[b] != -INFINITY) ? m[b] : 0.0f, l[b], pb[b]);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        // LDS reads issued after block db's: the window's later blocks
        constexpr int after_cap = 2 * (VW - 1);
        if (7 - db >= VW - 1) lds_wait_n<after_cap>(va[db], vb[db]);
        else if (7 - db == 2) lds_wait_n<4>(va[db], vb[db]);
        else if (7 - db == 1) lds_wait_n<2>(va[db], vb[db]);
        else lds_wait_n<0>(va[db], vb[db]);
        const bf16x8 vop = __builtin_shufflevector(va[db], vb[db], 0, 1, 2, 3, 4, 5, 6, 7);
        if (db + VW < 8) {
            va[db + VW] = ds_read_tr16_b64_at<VOFF>(vrow0 + 16 * ((2 * (db + VW)) ^ sw0));
            vb[db + VW] = ds_read_tr16_b64_at<VOFF + 16 * S::ROWB>(vrow0 + 16 * ((2 * (db + VW)) ^ sw0));
        }
#pragma unroll
        for (int b = 0; b < NBA; ++b) o[b][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[b], vop, o[b][db], 0, 0, 0);
    }
}

// Row maxima of one tile (log2 units), folded into m: exact pass only.
template <class S, int NBA, bool MASKED>
__device__ __forceinline__ void tile_max(const SplitArgs& a, const Ctx& cx, int tt, float c, const bf16x8 (&kop)[2][4],
                                         const bf16x8 (&qop)[NBA][4], float (&m)[NBA]) {
#pragma unroll
    for (int b = 0; b < NBA; ++b) {
        f32x4 sc[2];
        s_init<S, MASKED>(a, cx, tt, b, sc);
        qk_block(kop, qop[b], sc);
        const float m0 = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
        const float m1 = fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3]));
        m[b] = fmaxf(m[b], quad_max(fmaxf(m0, m1)) * c);
    }
}

// The work of one wavefront owning NBA query blocks.  SH: 0 normally; in the
// shared-block arrangement (13 query blocks on the (8,8,2) shape, where whole
// blocks would load the SIMDs 4/3/3/3) the last block belongs to no row
// group: waves 4-7 (one per SIMD, one block of their own each) take it on
// every fourth key tile each, and their four partial results meet in LDS at
// the end.  SH = 2 for those waves, 1 for the others (which only keep the
// barrier sequence).
template <class S, int LAYOUT, int NBA, bool EMIT, int SH = 0>
__device__ __forceinline__ void run_wave(const SplitArgs& a, const Ctx& cx) {
    constexpr int STAGES = S::STAGES;
    const float c = a.scale_log2;

    const int n = cx.n_tiles;
    // Q^T as the B operand: lane (li, lj) holds query row li of the block,
    // head-dim elements 32*s + 8*lj .. +7.  Rows past M repeat the first row
    // of this head group (their results are never stored).
    // own blocks 0 .. NBA-1, then (SH == 2) the shared block at index NBA
    constexpr int NBS = NBA + (SH == 2 ? 1 : 0);
    bf16x8 qop[NBS][4];
#pragma unroll
    for (int b = 0; b < NBA; ++b) {
        const int r = (cx.rg + b * S::R) * 16 + cx.li;
        const bool ok = r < a.M;
        const int t = ok ? r / a.G : 0;
        const int h = cx.g * a.G + (ok ? r % a.G : 0);
        const bf16x8* src = (const bf16x8*)(cx.q + ((size_t)t * a.Hq + h) * 128 + 8 * cx.lj);
#pragma unroll
        for (int s = 0; s < 4; ++s) qop[b][s] = src[4 * s];
    }
    // The fast pass's first load group goes out right behind the Q loads;
    // the wait below lets exactly those tile loads stay in flight, so the Q
    // latency hides under the first group's and the tile loop never waits
    // on Q.
    if (n >= S::GT) {
#pragma unroll
        for (int s = 0; s < S::GT; ++s) issue_tile<S, LAYOUT>(a, cx, s, s);
        wait_vmcnt<S::GT * S::NI>();
    } else {
#pragma unroll
        for (int s = 0; s < S::GT; ++s)
            if (s < n) issue_tile<S, LAYOUT>(a, cx, s, s);
        wait_vmcnt<0>();
    }

    float m_run[NBS], l_run[NBS];
    f32x4 o[NBS][8];
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
        m_run[b] = 0.0f;
        l_run[b] = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[b][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 kop[2][4], vop[8];

    // the shared block (SH == 2): a context whose row group names it (block
    // index rg + 0 * R), its Q operands at index NBA
    Ctx cxs = cx;
    cxs.rg = ((a.M + 15) >> 4) - 1;
    const int sh_k = cx.w - 4;                   // this wave's share: tiles t with t % 4 == sh_k
    if constexpr (SH == 2) {
        const int r = cxs.rg * 16 + cx.li;
        const bool ok = r < a.M;
        const int t = ok ? r / a.G : 0;
        const int h = cx.g * a.G + (ok ? r % a.G : 0);
        const bf16x8* src = (const bf16x8*)(cx.q + ((size_t)t * a.Hq + h) * 128 + 8 * cx.lj);
#pragma unroll
        for (int s = 0; s < 4; ++s) qop[NBS - 1][s] = src[4 * s];
    }
    // views of the own blocks, and of the shared block alone
    auto& qown = *reinterpret_cast<bf16x8 (*)[NBA][4]>(&qop[0]);
    auto& mown = *reinterpret_cast<float (*)[NBA]>(&m_run[0]);
    auto& lown = *reinterpret_cast<float (*)[NBA]>(&l_run[0]);
    auto& oown = *reinterpret_cast<f32x4 (*)[NBA][8]>(&o[0]);
    auto& qsh = *reinterpret_cast<bf16x8 (*)[1][4]>(&qop[NBS - 1]);
    auto& msh = *reinterpret_cast<float (*)[1]>(&m_run[NBS - 1]);
    auto& lsh = *reinterpret_cast<float (*)[1]>(&l_run[NBS - 1]);
    auto& osh = *reinterpret_cast<f32x4 (*)[1][8]>(&o[NBS - 1]);

    // One pass over the split's tiles; every pass crosses one barrier per
    // load group (plus one at the start of a rerun), identically in all
    // waves.
    //   FAST: p = 2^(s*c);  MAXONLY: exact row maxima;  EXACT: p = 2^(s*c - m).
    // The fast pass's first tiles are already in flight.
    constexpr int FAST = 0, MAXONLY = 1, EXACT = 2;
    auto pass = [&](auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
        if constexpr (MODE != FAST) {
            // no wave may refill the ring while another still reads the
            // previous pass's last tile
            barrier_lds();
#pragma unroll
            for (int s = 0; s < S::GT; ++s)
                if (s < n) issue_tile<S, LAYOUT>(a, cx, s, s);
        }
        // Full prefix tiles come first; the ragged end of the slice and the
        // tree's own rows (masked) come last, so the two kinds run in
        // separate loops with one copy of the tile code each.
        const int n_full = (int)((cx.c1 - cx.c0) / S::TK);
        auto group_start = [&](int t) {
            // The group starting at tile t is the only one in flight.
            wait_vmcnt<0>();
            barrier_lds();
            // The previous group's stages are free once every wave passed
            // the barrier; the next group goes into them.
#pragma unroll
            for (int j = 0; j < S::GT; ++j)
                if (t + S::GT + j < n) issue_tile<S, LAYOUT>(a, cx, t + S::GT + j, (t + S::GT + j) % STAGES);
        };
        // One tile from stage Ks + SOFF.
        auto tile = [&](int t, const char* Ks, auto masked_c, auto soff_c) {
            constexpr bool MASKED = decltype(masked_c)::value;
            constexpr int SOFF = decltype(soff_c)::value;
            if constexpr (MODE == MAXONLY) {
                load_k<S, SOFF>(Ks, cx, kop);
                tile_max<S, NBA, MASKED>(a, cx, t, c, kop, qown, mown);
                if constexpr (SH == 2)
                    if ((t & 3) == sh_k) tile_max<S, 1, MASKED>(a, cxs, t, c, kop, qsh, msh);
            } else if constexpr (S::WAVES == 8) {
                if constexpr (SH == 2 && !MASKED) {
                    // an unmasked tile does not need the blocks' row
                    // indices, so on this wave's share the shared block runs
                    // as one more block of the same tile
                    if ((t & 3) == sh_k) {
                        tile_pv_shared<S, NBS, false, MODE == EXACT, false, SOFF>(a, cx, t, c, Ks, qop, m_run, l_run,
                                                                                  o);
                        return;
                    }
                }
                tile_pv_shared<S, NBA, MASKED, MODE == EXACT, EMIT && MODE == FAST, SOFF>(a, cx, t, c, Ks, qown, mown,
                                                                                         lown, oown);
                if constexpr (SH == 2 && MASKED)
                    if ((t & 3) == sh_k)
                        tile_pv_shared<S, 1, true, MODE == EXACT, false, SOFF>(a, cxs, t, c, Ks, qsh, msh, lsh, osh);
            } else {
                load_k<S, SOFF>(Ks, cx, kop);
                load_v<S, SOFF>(Ks, cx, vop);
                tile_pv<S, NBA, MASKED, MODE == EXACT, EMIT && MODE == FAST>(a, cx, t, c, kop, vop, qop, m_run,
                                                                            l_run, o);
            }
        };
        using Unmasked = std::false_type;
        using Masked = std::true_type;
        int t = 0;
        // Whole groups of full tiles: the group's tiles are unrolled so
        // their stage offsets are constants.
        // The next group goes out in two halves, at the start of this group
        // and half-way through it (32 KB per work-group at a time): a whole
        // group of 64 KB at once exceeds the LDS-DMA requests a CU keeps in
        // flight, and the issuing waves would stall until earlier requests
        // drain.
        constexpr int HALF = S::GT >= 2 ? S::GT / 2 : 1;
        auto issue_half = [&](int tn) {
#pragma unroll
            for (int j = 0; j < HALF; ++j)
                if (tn + j < n) issue_tile<S, LAYOUT>(a, cx, tn + j, (tn + j) % STAGES);
        };
        for (; t + S::GT <= n_full; t += S::GT) {
            const char* gb = cx.smem + (t % STAGES) * S::STAGE;
            // (the 17-24-block shape keeps the single burst: the split issue
            // pushes its registers into spills)
            if constexpr (S::R == 8 && S::NB >= 3) {
                group_start(t);
                tile(t, gb, Unmasked{}, std::integral_constant<int, 0>{});
                if constexpr (S::GT >= 2) tile(t + 1, gb, Unmasked{}, std::integral_constant<int, S::STAGE>{});
                if constexpr (S::GT >= 4) {
                    tile(t + 2, gb, Unmasked{}, std::integral_constant<int, 2 * S::STAGE>{});
                    tile(t + 3, gb, Unmasked{}, std::integral_constant<int, 3 * S::STAGE>{});
                }
                continue;
            }
            wait_vmcnt<0>();
            barrier_lds();
            issue_half(t + S::GT);
            tile(t, gb, Unmasked{}, std::integral_constant<int, 0>{});
            if constexpr (S::GT == 2) {
                issue_half(t + S::GT + HALF);
                tile(t + 1, gb, Unmasked{}, std::integral_constant<int, S::STAGE>{});
            }
            if constexpr (S::GT == 4) {
                tile(t + 1, gb, Unmasked{}, std::integral_constant<int, S::STAGE>{});
                issue_half(t + S::GT + HALF);
                tile(t + 2, gb, Unmasked{}, std::integral_constant<int, 2 * S::STAGE>{});
                tile(t + 3, gb, Unmasked{}, std::integral_constant<int, 3 * S::STAGE>{});
            }
        }
        static_assert(S::GT == 1 || S::GT == 2 || S::GT == 4, "load group size");
        for (; t < n_full; ++t) {
            if (t % S::GT == 0) group_start(t);
            tile(t, cx.smem + (t % STAGES) * S::STAGE, Unmasked{}, std::integral_constant<int, 0>{});
        }
        for (; t < n; ++t) {
            if (t % S::GT == 0) group_start(t);
            tile(t, cx.smem + (t % STAGES) * S::STAGE, Masked{}, std::integral_constant<int, 0>{});
        }
    };

    pass(std::integral_constant<int, FAST>{});

    // The KS key sub-tiles of each row group meet through LDS.  Every wave
    // of the row group finishes DPW = 8/KS of the 8 column blocks of each
    // block (wave ks: column blocks ks*DPW ..), so the work is spread over
    // all KS waves; the others' sums for those columns and every wave's
    // per-row (m, l) are parked in LDS first (the exchange region overlaps
    // the ring, hence the barrier before).  The partial sums are added in
    // sub-tile order 0..KS-1 whichever wave finishes, so the result does not
    // depend on the assignment.
    f32x4* xo = (f32x4*)cx.smem;
    float* xml = (float*)(cx.smem + S::XO_BYTES);
    // parked column k (0 .. 8-DPW-1) of source wave src: column block db of
    // src, skipping src's own range
    auto xo_at = [&](int b, int src, int k) {
        return xo + ((((cx.rg * S::NB + b) * S::KS + src) * (8 - S::DPW) + k) * 64 + cx.lane);
    };
    auto xml_at = [&](int b, int src) { return xml + ((cx.rg * S::NB + b) * S::KS + src) * 32; };
    // the shared block's exchange: the four partial O (8 column blocks per
    // lane) from the start of the ring, then per-row (m, l)
    f32x4* sxo = (f32x4*)cx.smem;
    float* sxml = (float*)(cx.smem + 4 * 8 * 64 * 16);
    auto park = [&]() {
        // row sums: each lane summed its own keys; add the four lane groups
#pragma unroll
        for (int b = 0; b < NBA; ++b) l_run[b] = quad_sum(l_run[b]);
        if constexpr (SH != 0) {
            if constexpr (SH == 2) lsh[0] = quad_sum(lsh[0]);
            barrier_lds();                       // the ring is free
            if constexpr (SH == 2) {
#pragma unroll
                for (int db = 0; db < 8; ++db) sxo[(sh_k * 8 + db) * 64 + cx.lane] = osh[0][db];
                if (cx.lj == 0) {
                    sxml[sh_k * 32 + cx.li] = msh[0];
                    sxml[sh_k * 32 + 16 + cx.li] = lsh[0];
                }
            }
            barrier_lds();
        }
        if constexpr (S::KS > 1) {
            barrier_lds();
#pragma unroll
            for (int b = 0; b < NBA; ++b) {
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const int owner = db / S::DPW;
                    if (owner == cx.ks) continue;
                    *xo_at(b, cx.ks, db < cx.ks * S::DPW ? db : db - S::DPW) = o[b][db];
                }
                if (cx.lj == 0) {
                    xml_at(b, cx.ks)[cx.li] = m_run[b];
                    xml_at(b, cx.ks)[16 + cx.li] = l_run[b];
                }
            }
            barrier_lds();
        }
    };
    park();

    // Accept the fast pass only if, for every row of the work-group, the sum
    // of p over all its key sub-tiles (from the parked sums: one wave's share
    // of a row may legitimately hold no visible key) is finite and not
    // vanishing (a split with any tile gives every row at least one visible
    // key), and the accumulators are finite.
    int* votes = (int*)(cx.smem + S::SMEM);
    bool bad = false;
#pragma unroll
    for (int b = 0; b < NBA; ++b) {
        float os = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) os += (o[b][db][0] + o[b][db][1]) + (o[b][db][2] + o[b][db][3]);
        bad = bad || !(os - os == 0.0f);
    }
    if (n > 0) {
#pragma unroll
        for (int b = 0; b < NBA; ++b) {
            float L = 0.0f;
            if constexpr (S::KS > 1) {
#pragma unroll
                for (int k2 = 0; k2 < S::KS; ++k2) L += xml_at(b, k2)[16 + cx.li];
            } else {
                L = l_run[b];                        // every lane (li, lj) holds row li's sum
            }
            bad = bad || !(L >= kMinRowSum && L <= 3.0e38f);
        }
        if constexpr (SH == 2) {
            // the shared block's rows over all four shares (the fast pass
            // has m = 0 in every share, so the sums add up)
            float L = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) L += sxml[k * 32 + 16 + cx.li];
            bad = bad || !(L >= kMinRowSum && L <= 3.0e38f);
        }
    }
    if constexpr (SH == 2) {
        float os = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) os += (osh[0][db][0] + osh[0][db][1]) + (osh[0][db][2] + osh[0][db][3]);
        bad = bad || !(os - os == 0.0f);
    }
    // Work-group vote: a flagged wave sends every wave through the exact
    // path, which keeps the barrier sequence identical across waves.
    if (cx.lane == 0) votes[cx.w] = __builtin_amdgcn_ballot_w64(bad) != 0;
    barrier_lds();
    int any_vote = 0;
#pragma unroll
    for (int v = 0; v < S::WAVES; ++v) any_vote |= votes[v];
    if (any_vote) {
#pragma unroll
        for (int b = 0; b < NBA; ++b) m_run[b] = -INFINITY;
        msh[0] = -INFINITY;
        pass(std::integral_constant<int, MAXONLY>{});
#pragma unroll
        for (int b = 0; b < NBA; ++b) {
            l_run[b] = 0.0f;
#pragma unroll
            for (int db = 0; db < 8; ++db) o[b][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        lsh[0] = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) osh[0][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        pass(std::integral_constant<int, EXACT>{});
        park();
    }

    if constexpr (SH == 2) {
        // The shared block: wave 4 + k finishes column blocks 2k, 2k+1 from
        // the four parked shares, added in share order; wave 4 writes the LSE.
        // Weights per row: w_j = 2^(m_j - max m) (0 for a share without a
        // visible key), L = sum w_j l_j.
        const int rbase = cxs.rg * 16;
        auto share_w = [&](int row, float (&wj)[4], float& mmax, float& L) {
            float mj[4], lj[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mj[j] = sxml[j * 32 + row];
                lj[j] = sxml[j * 32 + 16 + row];
            }
            mmax = fmaxf(fmaxf(mj[0], mj[1]), fmaxf(mj[2], mj[3]));
            L = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wj[j] = mj[j] == -INFINITY ? 0.0f : exp2_fast(mj[j] - mmax);
                L += wj[j] * lj[j];
            }
        };
        if (sh_k == 0 && cx.lj == 0 && rbase + cx.li < a.M) {
            float wj[4], mmax, L;
            share_w(cx.li, wj, mmax, L);
            const int r = rbase + cx.li;
            const size_t orow = ((size_t)cx.row0 + r / a.G) * a.Hq + cx.g * a.G + r % a.G;
            a.part_lse[orow] = L > 0.0f ? (mmax + __log2f(L)) * kLn2 : -INFINITY;
        }
        float wq[4][4];
        float* dst[4];
        bool row_ok[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = 4 * cx.lj + i;
            float wj[4], mmax, L;
            share_w(q, wj, mmax, L);
            const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) wq[i][j] = wj[j] * inv;
            const int r = rbase + q;
            row_ok[i] = r < a.M;
            const int rr = row_ok[i] ? r : rbase;
            const size_t orow = ((size_t)cx.row0 + rr / a.G) * a.Hq + cx.g * a.G + rr % a.G;
            dst[i] = a.part_o + orow * 128 + cx.li;
        }
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) {
            const int db = 2 * sh_k + d2;
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 x = sxo[(j * 8 + db) * 64 + cx.lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += wq[i][j] * x[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (row_ok[i]) dst[i][16 * db] = acc[i];
        }
    }

#pragma unroll
    for (int b = 0; b < NBA; ++b) {
        // per-row weights of the KS partial sums, computed by the lanes that
        // own row li, in sub-tile order
        float mk[S::KS], lk[S::KS];
#pragma unroll
        for (int k = 0; k < S::KS; ++k) {
            if constexpr (S::KS > 1) {
                mk[k] = xml_at(b, k)[cx.li];
                lk[k] = xml_at(b, k)[16 + cx.li];
            } else {
                mk[k] = m_run[b];
                lk[k] = l_run[b];
            }
        }
        float mmax = mk[0];
#pragma unroll
        for (int k = 1; k < S::KS; ++k) mmax = fmaxf(mmax, mk[k]);
        float wk[S::KS];
        float L = 0.0f;
#pragma unroll
        for (int k = 0; k < S::KS; ++k) {
            wk[k] = mk[k] == -INFINITY ? 0.0f : exp2_fast(mk[k] - mmax);
            L += wk[k] * lk[k];
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const int rbase = (cx.rg + b * S::R) * 16;
        if (cx.ks == 0 && cx.lj == 0 && rbase + cx.li < a.M) {
            const int r = rbase + cx.li;
            const size_t orow = ((size_t)cx.row0 + r / a.G) * a.Hq + cx.g * a.G + r % a.G;
            a.part_lse[orow] = L > 0.0f ? (mmax + __log2f(L)) * kLn2 : -INFINITY;
        }
        // accumulator element i of this lane belongs to row 4*lj + i; the
        // per-row weights and destinations are formed once
        float wq[4][S::KS];
        float* dst[4];
        bool row_ok[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = 4 * cx.lj + i;
#pragma unroll
            for (int k = 0; k < S::KS; ++k) wq[i][k] = __shfl(wk[k] * inv, q);
            const int r = rbase + q;
            row_ok[i] = r < a.M;
            const int rr = row_ok[i] ? r : rbase;
            const size_t orow = ((size_t)cx.row0 + rr / a.G) * a.Hq + cx.g * a.G + rr % a.G;
            dst[i] = a.part_o + orow * 128 + cx.li;
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            if (db / S::DPW != cx.ks) continue;
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < S::KS; ++k) {
                const f32x4 x = k == cx.ks ? o[b][db] : *xo_at(b, k, db < k * S::DPW ? db : db - S::DPW);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += wq[i][k] * x[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (row_ok[i]) dst[i][16 * db] = acc[i];
        }
    }
}

template <int W, int R, int NB, int MODE_ARG>
__global__ __launch_bounds__(W * 64, 1) void split_mfma(const SplitArgs a) {
    // the root-score variant streams keys exactly as the contiguous layout
    constexpr int MODE = MODE_ARG == kModeContigRoot ? kModeContig : MODE_ARG;
    constexpr bool EMIT = MODE_ARG == kModeContigRoot;
    using S = Shape<W, R, NB, MODE>;
    constexpr int SMEM = S::SMEM;
    constexpr int MASK_OFF = (SMEM + S::POOL + 7) & ~7;
    static_assert(MASK_OFF + 64 * 8 <= 160 * 1024, "LDS budget");
    static_assert(S::NI >= 1 && (S::TK / 2) % S::WAVES == 0, "tile / wave split");
    // + the votes used once after the fast pass, + the tree mask
    // (read from LDS in masked tiles: a per-lane read of the kernel
    // arguments would be a vector memory load, and waiting for it would
    // drain the K/V ring)
    __shared__ __attribute__((aligned(1024))) char smem[MASK_OFF + 64 * 8];

    Ctx cx;
    cx.smem = smem;
    cx.lane = threadIdx.x & 63;
    cx.li = cx.lane & 15;
    cx.lj = cx.lane >> 4;
    // wave index as a scalar, so per-wave choices compile to scalar branches
    cx.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    cx.rg = cx.w / S::KS;
    cx.ks = cx.w % S::KS;
    cx.g = blockIdx.y;
    // paged batch: grid x enumerates every sequence's splits (a run per
    // sequence, as many as its length needs); otherwise x is the split
    int b = 0;
    cx.split = blockIdx.x;
    int seq_splits = a.n_splits;
    int64_t n_keys = a.n_keys;
    int64_t chunk = a.chunk_keys;
    cx.n_prefix = a.n_prefix;
    constexpr bool PAGED = MODE == kModePaged || MODE == kModePagedGather;
    if constexpr (PAGED) {
        while (b + 1 < a.B && (int)blockIdx.x >= a.seg_base[b + 1]) ++b;
        cx.split = blockIdx.x - a.seg_base[b];
        seq_splits = a.seg_base[b + 1] - a.seg_base[b];
        cx.n_prefix = a.npb[b];
        n_keys = MODE == kModePagedGather ? a.nib[b] : cx.n_prefix;
        chunk = (n_keys + seq_splits - 1) / seq_splits;
        chunk = (chunk + S::TK - 1) / S::TK * S::TK;
    }
    cx.q = (const __bf16*)a.q + (size_t)b * a.T * a.Hq * 128;
    cx.row0 = (int64_t)blockIdx.x * a.T;
    cx.c0 = (int64_t)cx.split * chunk;
    if (cx.c0 > n_keys) cx.c0 = n_keys;
    cx.c1 = cx.c0 + chunk < n_keys ? cx.c0 + chunk : n_keys;
    cx.n_pre_tiles = cx.c1 > cx.c0 ? (int)((cx.c1 - cx.c0 + S::TK - 1) / S::TK) : 0;
    const int n_tail_tiles = cx.split == seq_splits - 1 ? (a.T + S::TK - 1) / S::TK : 0;
    cx.n_tiles = cx.n_pre_tiles + n_tail_tiles;
    // paged: this head's rows start g * page_rows rows into every page
    const size_t head_off = PAGED ? (size_t)cx.g * a.page_rows * S::ROWB
                                               : (size_t)cx.g * (size_t)a.kv_head_stride * 2;
    cx.kbase = (const char*)a.k + head_off;
    cx.vbase = (const char*)a.v + head_off;
    // contiguous: the split's rows [c0, c1), and in the last split the tree
    // rows after the prefix (the host keeps this under 4 GB)
    cx.kseg = cx.kbase + cx.c0 * S::ROWB;
    cx.vseg = cx.vbase + cx.c0 * S::ROWB;
    cx.seg_bytes = (uint32_t)(((n_tail_tiles ? cx.n_prefix + a.T : cx.c1) - cx.c0) * S::ROWB);
    int32_t* idx_lds = (int32_t*)(smem + S::RING);
    cx.idx_lds = idx_lds;
    uint64_t* mask_lds = (uint64_t*)(smem + MASK_OFF);
    cx.mask_lds = mask_lds;
    // visible to all waves after the first barrier of the tile loop
    if (threadIdx.x < (unsigned)a.T) mask_lds[threadIdx.x] = a.mask[threadIdx.x];
    // the root-score variant also zeroes the counters its consumer
    // accumulates into (the kernel that runs before their first use)
    if constexpr (EMIT)
        if (a.root_clear && blockIdx.x == 0 && blockIdx.y == 0)
            for (int i = threadIdx.x; i < 1024; i += W * 64) a.root_clear[i] = 0u;
    cx.pg0 = cx.tpg0 = 0;
    cx.npg = 0;
    if constexpr (MODE == kModeGather) {
        const int n = (int)(cx.c1 > cx.c0 ? cx.c1 - cx.c0 : 0);
        for (int i = threadIdx.x; i < n; i += S::WAVES * 64) idx_lds[i] = a.idx[cx.c0 + i];
        __syncthreads();
    }
    if constexpr (MODE == kModePaged) {
        // the pages of this split's slice, then (last split) those of the
        // tree rows, from this sequence's row of the block table
        const int32_t* table = a.table + (size_t)b * a.table_stride;
        cx.pg0 = cx.c0 >> a.page_shift;
        cx.npg = cx.c1 > cx.c0 ? (int)(((cx.c1 - 1) >> a.page_shift) - cx.pg0 + 1) : 0;
        cx.tpg0 = cx.n_prefix >> a.page_shift;
        const int ntp = cx.split == seq_splits - 1
                            ? (int)(((cx.n_prefix + a.T - 1) >> a.page_shift) - cx.tpg0 + 1) : 0;
        for (int i = threadIdx.x; i < cx.npg; i += S::WAVES * 64) idx_lds[i] = table[cx.pg0 + i];
        for (int i = threadIdx.x; i < ntp; i += S::WAVES * 64) idx_lds[cx.npg + i] = table[cx.tpg0 + i];
        __syncthreads();
    }
    if constexpr (MODE == kModePagedGather) {
        // this split's index slice and (last split) the tree rows, each
        // position translated to its pool row through the block table
        const int32_t* table = a.table + (size_t)b * a.table_stride;
        const int32_t* list = a.idx + (size_t)b * a.idx_stride;
        const int n = (int)(cx.c1 > cx.c0 ? cx.c1 - cx.c0 : 0);
        const uint32_t in_page = (uint32_t)(a.page_rows - 1);
        for (int i = threadIdx.x; i < n; i += S::WAVES * 64) {
            const uint32_t pos = (uint32_t)list[cx.c0 + i];
            idx_lds[i] = (int32_t)(((uint32_t)table[pos >> a.page_shift] << a.page_shift) | (pos & in_page));
        }
        if (cx.split == seq_splits - 1)
            for (int i = threadIdx.x; i < a.T; i += S::WAVES * 64) {
                const uint64_t pos = (uint64_t)cx.n_prefix + i;
                idx_lds[kGatherChunkMax + i] =
                    (int32_t)(((uint32_t)table[pos >> a.page_shift] << a.page_shift) | ((uint32_t)pos & in_page));
            }
        __syncthreads();
    }

    // Query blocks are dealt round-robin to the R row groups, so a wave owns
    // NB or NB-1 of them (the planner guarantees it).
    const int nblk = (a.M + 15) >> 4;
    const int nb_act = (nblk - cx.rg + S::R - 1) / S::R;
    if constexpr (S::R == 1) {
        run_wave<S, MODE, NB, EMIT>(a, cx);
    } else {
        if constexpr (S::R == 8 && S::NB == 2) {
            // 13 blocks: whole blocks would load the SIMDs 4/3/3/3; the last
            // one is shared by waves 4-7 instead (row groups 0-3 keep two)
            if (nblk == 13) {
                if (cx.rg < 4) run_wave<S, MODE, 2, EMIT, 1>(a, cx);
                else run_wave<S, MODE, 1, EMIT, 2>(a, cx);
                return;
            }
        }
        if (nb_act >= NB) run_wave<S, MODE, NB, EMIT>(a, cx);
        else run_wave<S, MODE, NB - 1, EMIT>(a, cx);
    }
}

template <int W, int R, int NB>
hipError_t launch(int mode, const SplitArgs& a, int n_kv_heads, hipStream_t stream) {
    // paged: n_splits counts the splits of all sequences
    const dim3 grid(a.n_splits, n_kv_heads);
    if (mode == kModeGather)
        hipLaunchKernelGGL((split_mfma<W, R, NB, kModeGather>), grid, dim3(W * 64), 0, stream, a);
    else if (mode == kModePaged)
        hipLaunchKernelGGL((split_mfma<W, R, NB, kModePaged>), grid, dim3(W * 64), 0, stream, a);
    else if (mode == kModePagedGather)
        hipLaunchKernelGGL((split_mfma<W, R, NB, kModePagedGather>), grid, dim3(W * 64), 0, stream, a);
    else if (mode == kModeContigRoot) {
        // no root-score variant of the 17-24-block shape (the host never asks)
        if constexpr (R == 8 && NB >= 3) return hipErrorInvalidValue;
        else hipLaunchKernelGGL((split_mfma<W, R, NB, kModeContigRoot>), grid, dim3(W * 64), 0, stream, a);
    }
    else
        hipLaunchKernelGGL((split_mfma<W, R, NB, kModeContig>), grid, dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mfma
}  // namespace tsw
