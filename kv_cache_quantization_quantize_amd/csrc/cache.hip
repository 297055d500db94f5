// cache.hip -- the row-copy kernel of the KV cache: appending a decode
// step's token to every slab's fp16 residual ring, and moving the fp16 tail
// of a prompt into the rings ([Metal post] "What we're actually optimizing":
// the newest residual_length tokens stay fp16).
//
// One launch moves keys and values (blockIdx.y); each lane moves 16 bytes,
// head_dim/8 lanes one token row (16 lanes at head_dim 128), so a wave
// covers whole rows with fully coalesced loads and stores.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

__global__ __launch_bounds__(256) void copy_rows_kernel(const RowCopy k, const RowCopy v, int64_t slabs,
                                                        int64_t n_rows, int D)
{
    const RowCopy& c = blockIdx.y == 0 ? k : v;
    const int kLanesPerRow = D / 8;                    // head_dim is a multiple of 16
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = slabs * n_rows * kLanesPerRow;
    if (i >= total) return;
    const int64_t lane = i % kLanesPerRow;
    const int64_t row_all = i / kLanesPerRow;
    const int64_t slab = row_all / n_rows;
    const int64_t row = row_all - slab * n_rows;
    const uint4* src = reinterpret_cast<const uint4*>(c.src + slab * c.src_bh_stride + row * D) + lane;
    uint4* dst = reinterpret_cast<uint4*>(c.dst + slab * c.dst_bh_stride + row * D) + lane;
    *dst = *src;
}

hipError_t launch_copy_rows(const RowCopy& k, const RowCopy& v, int64_t slabs, int64_t n_rows, int D,
                            hipStream_t stream) {
    const int64_t total = slabs * n_rows * (D / 8);
    const dim3 grid(static_cast<uint32_t>((total + 255) / 256), 2);
    hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(256), 0, stream, k, v, slabs, n_rows, D);
    return hipGetLastError();
}

}  // namespace kivi
