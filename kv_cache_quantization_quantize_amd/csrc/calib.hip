// calib.hip -- streaming kernels that measure the achievable HBM bandwidth
// on the running GPU (the VeloxQuant-MLX "Benchmarks" page, "KV-Cache Kernel
// Roofline: What Actually Limits Decode", calibrates its roofline on the
// hardware itself instead of the spec sheet).  Four traffic shapes, one per
// kernel a hot-path kernel is compared with:
//   copy   read n bytes, write n bytes;
//   read   read n bytes (the decode attend's shape: it writes almost nothing);
//   write  write n bytes;
//   mix    read n bytes, write 3n/8 bytes: the 4-bit flush's shape (2 B of
//          fp16 in for 0.5 B of codes + 0.25 B of scale/zero per element).
// Workgroup b owns one contiguous chunk; every thread issues all of its
// 16-byte loads before its first store.  Each kernel uses the cache hints
// and the residency that measured fastest for its shape on MI355X
// (interleaved runs over 2 GiB, three rounds each):
//  - the nontemporal hint on loads and stores for copy, read and mix (each
//    byte is touched once, as in the flush and the attend; plain stores made
//    the mix 10% slower and plain loads the read 17% slower), plain stores
//    for the write-only kernel (6.0-6.3 TB/s against 5.7-5.8 with the hint);
//  - fewer resident workgroups than the registers allow: each launch
//    reserves LDS it never touches so that only k workgroups of 4 waves fit
//    on a CU.  Unlimited (8+ per CU) the mix ran at 5.84-6.07 TB/s, the copy
//    at 5.8-6.1 and the write at 6.2-6.25; with k = 5, 4 and 3 they ran at
//    6.1-6.24, 6.22-6.25 and 6.57-6.67, and the read at k = 3 at 7.03-7.08
//    (6.86-6.94 unlimited).  Too few (3 per CU for the copy) loses again:
//    4.43-4.46 TB/s.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

namespace {

constexpr int kCalibBlock = 256;
constexpr int kCalibVecs = 4;                       // 16-byte vectors per thread per kernel
constexpr int64_t kCalibChunk = int64_t{kCalibBlock} * kCalibVecs;   // vectors per workgroup

// LDS a launch reserves so that at most k of its workgroups are resident on
// a CU (160 KiB of LDS per CU on gfx950).
constexpr size_t kLdsPerCU = 160 * 1024;
constexpr size_t lds_for(int per_cu) { return kLdsPerCU / per_cu; }
constexpr size_t kCopyLds = lds_for(4);
constexpr size_t kReadLds = lds_for(3);
constexpr size_t kWriteLds = lds_for(3);
constexpr size_t kMixLds = lds_for(5);

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u ld_nt(const v4u* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(v4u* p, v4u v) { __builtin_nontemporal_store(v, p); }

__global__ __launch_bounds__(kCalibBlock) void calib_copy_kernel(const v4u* __restrict__ src,
                                                                 v4u* __restrict__ dst, int64_t n_vec)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCalibChunk + threadIdx.x;
    v4u v[kCalibVecs];
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        if (i < n_vec) v[u] = ld_nt(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        if (i < n_vec) st_nt(dst + i, v[u]);
    }
}

// The loads are folded into one word that is stored only when it equals
// `never` (a value the caller picks; a chance match writes one word).
__global__ __launch_bounds__(kCalibBlock) void calib_read_kernel(const v4u* __restrict__ src, int64_t n_vec,
                                                                 uint32_t* __restrict__ sink, uint32_t never)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCalibChunk + threadIdx.x;
    v4u v[kCalibVecs];
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        v[u] = i < n_vec ? ld_nt(src + i) : v4u{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (acc == never) sink[0] = acc;
}

__global__ __launch_bounds__(kCalibBlock) void calib_write_kernel(v4u* __restrict__ dst, int64_t n_vec,
                                                                  uint32_t pattern)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCalibChunk + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        if (i < n_vec) dst[i] = v4u{pattern, pattern ^ static_cast<uint32_t>(i), pattern, 0u};
    }
}

// Workgroup b reads source vectors [b*C, (b+1)*C) and writes destination
// vectors [b*3C/8, (b+1)*3C/8), C = kCalibChunk: each wave writes 3/8 of what
// it loaded (the fold of its loads), as each flush wave writes its own tile.
__global__ __launch_bounds__(kCalibBlock) void calib_mix_kernel(const v4u* __restrict__ src, int64_t n_vec,
                                                                v4u* __restrict__ dst)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCalibChunk + threadIdx.x;
    v4u v[kCalibVecs];
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        v[u] = i < n_vec ? ld_nt(src + i) : v4u{0u, 0u, 0u, 0u};
    }
    v4u acc = v[0];
#pragma unroll
    for (int u = 1; u < kCalibVecs; ++u) acc ^= v[u];
    constexpr int kPerWave = 64 * kCalibVecs * 3 / 8;            // vectors a wave stores
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t o = static_cast<int64_t>(blockIdx.x) * (kCalibChunk * 3 / 8) + wave * kPerWave;
#pragma unroll
    for (int u = 0; u < (kPerWave + 63) / 64; ++u) {
        const int k = lane + 64 * u;
        const int64_t j = o + k;
        if (k < kPerWave && j < n_vec * 3 / 8) st_nt(dst + j, acc);
    }
}

uint32_t grid_of(int64_t n_vec) { return static_cast<uint32_t>((n_vec + kCalibChunk - 1) / kCalibChunk); }

}  // namespace

hipError_t launch_calib_copy(const void* src, void* dst, size_t n_bytes, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    hipLaunchKernelGGL(calib_copy_kernel, dim3(grid_of(n_vec)), dim3(kCalibBlock), kCopyLds, stream,
                       static_cast<const v4u*>(src), static_cast<v4u*>(dst), n_vec);
    return hipGetLastError();
}

hipError_t launch_calib_read(const void* src, size_t n_bytes, uint32_t* sink, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    hipLaunchKernelGGL(calib_read_kernel, dim3(grid_of(n_vec)), dim3(kCalibBlock), kReadLds, stream,
                       static_cast<const v4u*>(src), n_vec, sink, 0x9E3779B9u);
    return hipGetLastError();
}

hipError_t launch_calib_write(void* dst, size_t n_bytes, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    hipLaunchKernelGGL(calib_write_kernel, dim3(grid_of(n_vec)), dim3(kCalibBlock), kWriteLds, stream,
                       static_cast<v4u*>(dst), n_vec, 0x5A5A5A5Au);
    return hipGetLastError();
}

hipError_t launch_calib_mix(const void* src, size_t n_bytes, void* dst, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    hipLaunchKernelGGL(calib_mix_kernel, dim3(grid_of(n_vec)), dim3(kCalibBlock), kMixLds, stream,
                       static_cast<const v4u*>(src), n_vec, static_cast<v4u*>(dst));
    return hipGetLastError();
}

}  // namespace kivi
