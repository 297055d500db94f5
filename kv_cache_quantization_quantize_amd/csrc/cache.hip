// cache.hip -- the row-copy kernel of the KV cache: appending a decode
// step's token to every slab's fp16 residual ring, moving the fp16 tail of a
// prompt chunk into the rings, and assembling the token groups a chunk's
// flush takes partly from the ring and partly from the chunk ([Metal post]
// "What we're actually optimizing": the newest residual_length tokens stay
// fp16, older ones are flushed in whole groups).
//
// One launch moves keys and values (blockIdx.y).  Row r of a slab comes
// from span a (rows [0, n_a)) or span b (the rest) and goes to span dst;
// a span may be a ring, whose row index wraps.  Each lane moves 16 bytes,
// head_dim/8 lanes one token row (16 lanes at head_dim 128), so a wave
// covers whole rows with fully coalesced loads and stores.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

namespace {

__device__ __forceinline__ int64_t span_row(const RowSpan& s, int64_t r) {
    const int64_t i = s.first + r;
    return s.ring > 0 ? i % s.ring : i;
}

}  // namespace

__global__ __launch_bounds__(256) void gather_rows_kernel(const RowGather k, const RowGather v, int64_t slabs,
                                                          int64_t n_rows, int D)
{
    const RowGather& c = blockIdx.y == 0 ? k : v;
    const int kLanesPerRow = D / 8;                    // head_dim is a multiple of 16
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = slabs * n_rows * kLanesPerRow;
    if (i >= total) return;
    const int64_t lane = i % kLanesPerRow;
    const int64_t row_all = i / kLanesPerRow;
    const int64_t slab = row_all / n_rows;
    const int64_t row = row_all - slab * n_rows;
    const bool from_a = row < c.n_a;
    const RowSpan& s = from_a ? c.a : c.b;
    const int64_t srow = span_row(s, from_a ? row : row - c.n_a);
    const uint4* src = reinterpret_cast<const uint4*>(s.base + slab * s.bh_stride + srow * D) + lane;
    uint4* dst = reinterpret_cast<uint4*>(c.dst.base + slab * c.dst.bh_stride + span_row(c.dst, row) * D) + lane;
    *dst = *src;
}

hipError_t launch_gather_rows(const RowGather& k, const RowGather& v, int64_t slabs, int64_t n_rows, int D,
                              hipStream_t stream) {
    const int64_t total = slabs * n_rows * (D / 8);
    const dim3 grid(static_cast<uint32_t>((total + 255) / 256), 2);
    hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(256), 0, stream, k, v, slabs, n_rows, D);
    return hipGetLastError();
}

}  // namespace kivi
