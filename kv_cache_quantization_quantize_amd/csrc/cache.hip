// cache.hip -- the row-copy kernel of the KV cache: appending a decode
// step's token to every slab's fp16 residual ring, moving the fp16 tail of a
// prompt chunk into the rings, and assembling the token groups a chunk's
// flush takes partly from the ring and partly from the chunk ([Metal post]
// "What we're actually optimizing": the newest residual_length tokens stay
// fp16, older ones are flushed in whole groups).
//
// One launch moves keys and values (blockIdx.z).  Row r of a slab comes
// from span a (rows [0, n_a)) or span b (the rest) and goes to span dst;
// a span may be a ring, whose row index wraps.  Each lane moves 16 bytes,
// head_dim/8 lanes one token row (16 lanes at head_dim 128), so a wave
// covers whole rows with fully coalesced loads and stores.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

namespace {

// Row i of a span within one slab (row counts stay below 2^26, so 32-bit
// arithmetic suffices).
__device__ __forceinline__ int span_row(int first, int ring, int i) {
    const int r = first + i;
    return ring > 0 ? r % ring : r;
}

}  // namespace

// Grid: x covers the rows x lanes of one slab (lane = 16 bytes of a row),
// y strides over the slabs, z = 0 keys, 1 values.  LANES = head_dim / 8 for
// the common head_dims (shifts), 0 for a runtime count.  Each field of the
// gather is picked on its own (a scalar select), so nothing goes through
// private memory.
template <int LANES>
__global__ __launch_bounds__(256) void gather_rows_kernel(const RowGather k, const RowGather v, int64_t slabs,
                                                          int n_rows, int lanes_rt)
{
    const bool is_v = blockIdx.z != 0;
    const int lanes = LANES ? LANES : lanes_rt;
    const int idx = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
    if (idx >= n_rows * lanes) return;
    const int row = LANES ? idx / LANES : idx / lanes;
    const int lane = idx - row * lanes;
    const int D = lanes * 8;
    const int n_a = static_cast<int>(is_v ? v.n_a : k.n_a);
    const bool from_a = row < n_a;
    const RowSpan src = is_v ? (from_a ? v.a : v.b) : (from_a ? k.a : k.b);
    const RowSpan dst = is_v ? v.dst : k.dst;
    const int64_t srow = span_row(static_cast<int>(src.first), static_cast<int>(src.ring), from_a ? row : row - n_a);
    const int64_t drow = span_row(static_cast<int>(dst.first), static_cast<int>(dst.ring), row);
    for (int64_t slab = blockIdx.y; slab < slabs; slab += gridDim.y) {
        const uint4* from = reinterpret_cast<const uint4*>(src.base + slab * src.bh_stride + srow * D) + lane;
        uint4* to = reinterpret_cast<uint4*>(dst.base + slab * dst.bh_stride + drow * D) + lane;
        *to = *from;
    }
}

hipError_t launch_gather_rows(const RowGather& k, const RowGather& v, int64_t slabs, int64_t n_rows, int D,
                              hipStream_t stream) {
    const int lanes = D / 8;                           // head_dim is a multiple of 16
    const int64_t per_slab = n_rows * lanes;           // below 2^31: n_rows < 2^26, lanes <= 32
    const dim3 grid(static_cast<uint32_t>((per_slab + 255) / 256),
                    static_cast<uint32_t>(slabs < 65535 ? slabs : 65535), 2);
    const int nr = static_cast<int>(n_rows);
    switch (lanes) {
        case 8: hipLaunchKernelGGL(gather_rows_kernel<8>, grid, dim3(256), 0, stream, k, v, slabs, nr, lanes); break;
        case 16: hipLaunchKernelGGL(gather_rows_kernel<16>, grid, dim3(256), 0, stream, k, v, slabs, nr, lanes); break;
        case 32: hipLaunchKernelGGL(gather_rows_kernel<32>, grid, dim3(256), 0, stream, k, v, slabs, nr, lanes); break;
        default: hipLaunchKernelGGL(gather_rows_kernel<0>, grid, dim3(256), 0, stream, k, v, slabs, nr, lanes);
    }
    return hipGetLastError();
}

}  // namespace kivi
