// Device helpers shared by the gfx950 kernels (vector types, base-2
// exponential, cross-lane reductions, LDS swizzle, explicit waits).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace tsw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Shuffle-based reductions (ds_bpermute); any xor distance.
__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m)); }
__device__ __forceinline__ float xor_sum(float x, int m) { return x + __shfl_xor(x, m); }

// Combine lanes l, l^16, l^32, l^48 with the gfx950 permlane swaps (VALU,
// no LDS round trip).  After a swap of a value with itself, the two halves
// of the result hold x[l] and x[partner] in some order, so max/sum of the
// pair is the same in every lane.
__device__ __forceinline__ float quad_max(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16-byte chunk swizzles of 256-byte LDS rows: logical chunk c of tile row r
// lives in physical slot c ^ swz(r) (V rows) or c ^ swz_k(r) (K rows).
// V: for any 4 (and 8) consecutive aligned rows the chunk pairs {2b, 2b+1}
// land in different slot pairs, so the transposed V reads (two chunks of 4
// rows per 16 lanes) are free of bank conflicts.  K: a K operand read takes
// chunk 4s + lj of rows 0..15 (lane li, lj); with the slot XORed by the
// row's low four bits the read is conflict-free on gfx950, where the V
// swizzle cost it 4 conflict cycles per instruction (SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz(int r) { return ((2 * (r & 7)) | ((r >> 2) & 1)) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_k(int r) { return r & 15; }

// Cache policy for K/V rows that a call reads exactly once: the non-temporal
// (streaming) hint.  On MI355X it raises the aggregate LDS-DMA streaming rate
// of a one-work-group-per-CU kernel by 5-11% over the default policy.
constexpr int kStreamAux = 2;

// Raw buffer resource over `bytes` bytes from `base` (stride 0, 32-bit data
// format word): loads at offsets past the range return zeros and never
// fault, so a ragged tile needs no clamping of its row addresses.  For an
// LDS-DMA load the out-of-range dwords are written to LDS as zeros (checked
// on gfx950), so no stale LDS contents reach the products.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One LDS-DMA load of 16 bytes per lane from buffer r at voff + soff (bytes)
// into LDS at dst (uniform), with the streaming hint.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0,
                                             kStreamAux);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Transposed 64-bit LDS read (ds_read_b64_tr_b16) issued through inline
// assembly.  Through the builtin, the compiler puts s_waitcnt vmcnt(0) in
// front of every such read while LDS-DMA loads are outstanding, which would
// drain the whole K/V prefetch ring once per tile.  Here the compiler does not
// see the read: the caller must call lds_wait() on the results before use.
__device__ __forceinline__ bf16x4 ds_read_tr16_b64(const char* p) {
    bf16x4 r;
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
    return r;
}

// The same read at p + OFF, the constant in the instruction's offset field
// (no address arithmetic for it).
template <int OFF>
__device__ __forceinline__ bf16x4 ds_read_tr16_b64_at(const char* p) {
    static_assert(OFF >= 0 && OFF < 65536, "LDS instruction offset range");
    bf16x4 r;
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
    return r;
}

// Wait until at most N LDS operations are outstanding.  LDS reads complete
// in issue order, so with N = the number of LDS reads issued after x and y,
// x and y have landed (any other outstanding LDS operation only makes the
// wait stricter).
template <int N>
__device__ __forceinline__ void lds_wait_n(bf16x4& x, bf16x4& y) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "i"(N));
}

// Wait for every outstanding LDS read (and scalar load); tying the values
// keeps their uses after the wait.
__device__ __forceinline__ void lds_wait(bf16x4& x, bf16x4& y) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x), "+v"(y));
}

// Work-group barrier that does not wait for outstanding LDS-DMA loads (the
// pipelines wait for exactly the tiles they need with wait_vmcnt).  Pending
// LDS reads are drained first so a stage is never overwritten under a read.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace tsw
