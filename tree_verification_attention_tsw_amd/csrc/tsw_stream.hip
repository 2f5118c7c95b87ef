// Measurement aids, not steps of the method.
//
// Read-stream ceiling of the LDS-DMA path: streams every K and V row a tree-verification call reads,
// through the same kind of ring the matrix-core split kernel uses (two
// 128-key load groups of 64 KB per work-group, each issued in two 32 KB
// halves, one work-group per (split, kv head)), with no arithmetic.  Its
// rate is the HBM read rate the split kernel could reach if its compute
// were free.
#include "tsw_device.h"
#include "tsw_internal.h"

namespace tsw {
namespace {

constexpr int kStreamWaves = 8;
constexpr int kStreamTile = 64;                      // keys per half group
constexpr int kStreamTileBytes = 2 * kStreamTile * 256;   // K tile + V tile
constexpr int kStreamLoads = kStreamTile / 2 / kStreamWaves;  // 1 KB loads per wave per tile

// rows [c0, c1) of one kv head's K and V (256-byte rows; buffers krs / vrs
// start at row c0 and end at row c1), tile t into stage st; rows past c1
// read as zeros
__device__ __forceinline__ void stream_issue(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, int t, int st,
                                             char* smem, int w, int lane) {
    char* sbase = smem + st * kStreamTileBytes;
#pragma unroll
    for (int i = 0; i < kStreamLoads; ++i) {
        const int u = w * kStreamLoads + i;
        const bool isv = u >= kStreamTile / 4;
        const int grp = isv ? u - kStreamTile / 4 : u;
        const uint32_t off = (uint32_t)((grp * 4 + (lane >> 4)) * 256 + 16 * (lane & 15));
        char* dst = sbase + (isv ? kStreamTile * 256 : 0) + grp * 1024;
        buffer_load_lds16(isv ? vrs : krs, dst, off, (uint32_t)t * kStreamTile * 256);
    }
}

__global__ __launch_bounds__(kStreamWaves * 64, 1) void read_stream(const char* k, const char* v, int64_t head_bytes,
                                                                     int64_t rows, int64_t chunk, unsigned* sink) {
    __shared__ __attribute__((aligned(1024))) char smem[4 * kStreamTileBytes];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const char* kh = k + (int64_t)blockIdx.y * head_bytes;
    const char* vh = v + (int64_t)blockIdx.y * head_bytes;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int64_t c1 = c0 + chunk < rows ? c0 + chunk : rows;
    if (c0 >= c1) return;                                  // uniform: an empty split
    const int n = (int)((c1 - c0 + kStreamTile - 1) / kStreamTile);
    const __amdgpu_buffer_rsrc_t krs = raw_rsrc(kh + c0 * 256, (uint32_t)((c1 - c0) * 256));
    const __amdgpu_buffer_rsrc_t vrs = raw_rsrc(vh + c0 * 256, (uint32_t)((c1 - c0) * 256));
    // two groups of two tiles in the ring; a group's tiles are issued one
    // per tile of the group before it
    for (int t = 0; t < 2 && t < n; ++t) stream_issue(krs, vrs, t, t, smem, w, lane);
    unsigned acc = 0;
    for (int t = 0; t < n; t += 2) {
        wait_vmcnt<0>();
        barrier_lds();
        if (t + 2 < n) stream_issue(krs, vrs, t + 2, (t + 2) % 4, smem, w, lane);
        acc ^= *(volatile unsigned*)(smem + (t % 4) * kStreamTileBytes + threadIdx.x * 4);
        if (t + 3 < n) stream_issue(krs, vrs, t + 3, (t + 3) % 4, smem, w, lane);
        if (t + 1 < n) acc ^= *(volatile unsigned*)(smem + ((t + 1) % 4) * kStreamTileBytes + threadIdx.x * 4);
    }
    wait_vmcnt<0>();
    // never true for the caller's data in practice; keeps the reads alive
    if (acc == 0x9e3779b9u) sink[threadIdx.x & 15] = acc;
}

// Launch floor (a measurement aid): a kernel that does nothing, launched
// with a split kernel's grid, block and by-value arguments.
__global__ void launch_floor(const SplitArgs a) {
    if (a.n_splits < 0 && threadIdx.x == 0) a.part_lse[0] = 0.0f;   // never: keeps the argument live
}

}  // namespace

hipError_t launch_launch_floor(const SplitArgs& a, int n_kv_heads, int threads, hipStream_t stream) {
    hipLaunchKernelGGL(launch_floor, dim3(a.n_splits, n_kv_heads), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_read_stream(const void* k, const void* v, int n_kv_heads, int64_t head_bytes, int64_t rows,
                              int n_splits, unsigned* sink, hipStream_t stream) {
    const int64_t chunk = (rows + n_splits - 1) / n_splits;
    hipLaunchKernelGGL(read_stream, dim3(n_splits, n_kv_heads), dim3(kStreamWaves * 64), 0, stream,
                       (const char*)k, (const char*)v, head_bytes, rows, chunk, sink);
    return hipGetLastError();
}

}  // namespace tsw
