// calib.hip -- streaming kernels that measure the achievable HBM bandwidth
// on the running GPU (the VeloxQuant-MLX "Benchmarks" page, "KV-Cache Kernel
// Roofline: What Actually Limits Decode", calibrates its roofline on the
// hardware itself instead of the spec sheet).  Four traffic shapes, one per
// kernel a hot-path kernel is compared with:
//   copy   read n bytes, write n bytes;
//   read   read n bytes (the decode attend's shape: it writes almost nothing);
//   write  write n bytes;
//   mix    read n bytes, write 3n/8 bytes in the 4-bit flush's own pattern
//          (an 8 KiB tile read per wave; a quarter of it written to one
//          region and a sixteenth to each of two others, as codes, scales
//          and zeros).
// Every thread issues all of its 16-byte loads before its first store.  Each
// kernel uses the cache hints, the per-wave tile and the residency that
// measured fastest for its shape on MI355X (sweeps over 2 GiB after 200 ms
// of sustained load, three to five rounds each):
//  - the nontemporal hint on loads and stores for copy, read and mix (each
//    byte is touched once, as in the flush and the attend; plain stores made
//    the mix 10% slower and plain loads the read 17% slower), plain stores
//    for the write-only kernel (6.0-6.3 TB/s against 5.7-5.8 with the hint);
//  - fewer resident workgroups than the registers allow: each launch
//    reserves LDS it never touches so that only k workgroups of 4 waves fit
//    on a CU.  The read at k = 3 ran at 7.50-7.52 TB/s against 6.94-7.06
//    unlimited; the copy at k = 4 at 6.31-6.33 against 6.11-6.16 (4.48 at
//    k = 3); the write at k = 3 at 6.57-6.67 against 6.2;
//  - for the mix, the flush-shaped kernel at k = 3 ran at 6.51 TB/s median
//    (6.33-6.70), ahead of every plain streaming form tried (4 or 8 loads
//    per thread, block- or wave-contiguous, k from 3 to 8: at most 6.39).
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
constexpr size_t kMixLds = lds_for(3);

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

// The flush's own traffic without its arithmetic.  Wave t reads tile t,
// source vectors [512t, 512t + 512) (8 KiB: one 32-token x 128-channel fp16
// tile), and writes the fold of each lane's loads to three regions of dst,
// as the 4-bit flush writes codes, scales and zeros: 128 vectors (2 KiB) at
// codes[128t ..], 32 at scale[32t ..] and 32 at zero[32t ..].  The regions
// hold floor(n/4), floor(n/16) and the rest of floor(3n/8) vectors (n source
// vectors), so dst receives exactly floor(3n/8) vectors; the last tile's
// counts absorb a ragged end.
constexpr int kMixTile = 512;                       // source vectors per wave
constexpr int kMixWaves = kCalibBlock / 64;

__global__ __launch_bounds__(kCalibBlock) void calib_mix_kernel(const v4u* __restrict__ src, int64_t n_vec,
                                                                v4u* __restrict__ dst)
{
    const int lane = threadIdx.x & 63;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kMixWaves + (threadIdx.x >> 6);
    const int64_t n_tiles = (n_vec + kMixTile - 1) / kMixTile;
    if (tile >= n_tiles) return;                    // uniform across the wave
    const int64_t base = tile * kMixTile + lane;
    v4u v[kMixTile / 64];
#pragma unroll
    for (int u = 0; u < kMixTile / 64; ++u) {
        const int64_t i = base + u * 64;
        v[u] = i < n_vec ? ld_nt(src + i) : v4u{0u, 0u, 0u, 0u};
    }
    v4u acc = v[0];
#pragma unroll
    for (int u = 1; u < kMixTile / 64; ++u) acc ^= v[u];
    const int64_t m_codes = n_vec / 4, m_scale = n_vec / 16;
    const int64_t m_zero = n_vec * 3 / 8 - m_codes - m_scale;
    const bool last = tile == n_tiles - 1;
    const int64_t n_c = last ? m_codes - tile * 128 : 128;
    const int64_t n_s = last ? m_scale - tile * 32 : 32;
    const int64_t n_z = last ? m_zero - tile * 32 : 32;
    v4u* codes = dst + tile * 128;
    v4u* scale = dst + m_codes + tile * 32;
    v4u* zero = dst + m_codes + m_scale + tile * 32;
    for (int64_t k = lane; k < n_c; k += 64) st_nt(codes + k, acc);
    if (lane < 32) {
        for (int64_t k = lane; k < n_s; k += 32) st_nt(scale + k, acc);
    } else {
        for (int64_t k = lane - 32; k < n_z; k += 32) st_nt(zero + k, acc);
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
    const int64_t tiles = (n_vec + kMixTile - 1) / kMixTile;
    hipLaunchKernelGGL(calib_mix_kernel, dim3(static_cast<uint32_t>((tiles + kMixWaves - 1) / kMixWaves)),
                       dim3(kCalibBlock), kMixLds, stream,
                       static_cast<const v4u*>(src), n_vec, static_cast<v4u*>(dst));
    return hipGetLastError();
}

}  // namespace kivi
