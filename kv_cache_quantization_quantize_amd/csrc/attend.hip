// attend.hip -- the decode attend for fp16 caches (the partial kernel of
// attend_device.h; its split plan is in plan.cpp) and the log-sum-exp
// combine kernel that both the fp16 and the bfloat16 attends finish with.
#include <algorithm>

#include "attend_device.h"

namespace kivi {

// Merge the splits of one (sequence, query head), base-2 log-sum-exp:
// o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i with M = max_i m_i.
// Partials and out have ds channels (ds <= D, a multiple of 16).  WAVES
// waves per row: wave w takes splits w, w + WAVES, ..., lane l channels 2l
// and 2l + 1, and at head_dim 256 also 128 + 2l and 129 + 2l, where they
// lie below ds; the waves' sums meet in LDS.  The first kU splits of every
// wave are loaded together with their (m, l) before the maximum is known, so
// a row of up to kU * WAVES splits costs one memory round trip; only longer
// rows loop over the rest.
template <int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void attend_combine_kernel(const float* __restrict__ ws_o,
                                                                   const float* __restrict__ ws_ml,
                                                                   int64_t n_part, float* __restrict__ out,
                                                                   int ds)
{
    constexpr int kU = 4;
    constexpr int kV = D > 128 ? D / 128 : 1;        // channel pairs per lane
    __shared__ float red_m[WAVES];
    __shared__ float red_l[WAVES];
    __shared__ float2 red_o[WAVES][kV][64];
    const int64_t row = blockIdx.x;                  // b * Hq + h
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const float* ml = ws_ml + row * n_part * 2;
    const float2* o = reinterpret_cast<const float2*>(ws_o + row * n_part * ds) + l;
    bool has[kV];                                    // the lane's pair v lies below ds
#pragma unroll
    for (int v = 0; v < kV; ++v) has[v] = 2 * l + 128 * v < ds;

    float2 mv[kU], ov[kU][kV];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t i = w + static_cast<int64_t>(u) * WAVES;
        mv[u] = i < n_part ? *reinterpret_cast<const float2*>(ml + 2 * i) : make_float2(-INFINITY, 0.0f);
#pragma unroll
        for (int v = 0; v < kV; ++v)
            ov[u][v] = (i < n_part && has[v]) ? o[i * (ds / 2) + 64 * v] : make_float2(0.0f, 0.0f);
    }
    float M = mv[0].x;
#pragma unroll
    for (int u = 1; u < kU; ++u) M = fmaxf(M, mv[u].x);
    for (int64_t i = w + static_cast<int64_t>(kU) * WAVES; i < n_part; i += WAVES) M = fmaxf(M, ml[2 * i]);
    if (l == 0) red_m[w] = M;                        // uniform across the wave
    __syncthreads();
    M = red_m[0];
#pragma unroll
    for (int i = 1; i < WAVES; ++i) M = fmaxf(M, red_m[i]);
    // every partial empty (a sequence with no tokens): keep the weights finite (0)
    if (M == -INFINITY) M = 0.0f;

    float L = 0.0f;
    float2 acc[kV];
#pragma unroll
    for (int v = 0; v < kV; ++v) acc[v] = make_float2(0.0f, 0.0f);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const float e = exp2f(mv[u].x - M);
        L = __builtin_fmaf(e, mv[u].y, L);
#pragma unroll
        for (int v = 0; v < kV; ++v) {
            acc[v].x = __builtin_fmaf(e, ov[u][v].x, acc[v].x);
            acc[v].y = __builtin_fmaf(e, ov[u][v].y, acc[v].y);
        }
    }
    for (int64_t i = w + static_cast<int64_t>(kU) * WAVES; i < n_part; i += WAVES) {
        const float2 m2 = *reinterpret_cast<const float2*>(ml + 2 * i);
        const float e = exp2f(m2.x - M);
        L = __builtin_fmaf(e, m2.y, L);
#pragma unroll
        for (int v = 0; v < kV; ++v) {
            const float2 o2 = has[v] ? o[i * (ds / 2) + 64 * v] : make_float2(0.0f, 0.0f);
            acc[v].x = __builtin_fmaf(e, o2.x, acc[v].x);
            acc[v].y = __builtin_fmaf(e, o2.y, acc[v].y);
        }
    }
#pragma unroll
    for (int v = 0; v < kV; ++v) red_o[w][v][l] = acc[v];
    if (l == 0) red_l[w] = L;
    __syncthreads();
    if (w == 0) {
        float Lt = red_l[0];
#pragma unroll
        for (int u = 1; u < WAVES; ++u) Lt += red_l[u];
#pragma unroll
        for (int v = 0; v < kV; ++v) {
            float2 at = red_o[0][v][l];
#pragma unroll
            for (int u = 1; u < WAVES; ++u) {
                at.x += red_o[u][v][l].x;
                at.y += red_o[u][v][l].y;
            }
            // a sequence with no tokens at all (only possible in a variable-length
            // batch) has every partial empty (m = -inf, l = 0): its output is zero
            const float2 r = Lt > 0.0f ? make_float2(at.x / Lt, at.y / Lt) : make_float2(0.0f, 0.0f);
            if (has[v]) reinterpret_cast<float2*>(out + row * ds)[l + 64 * v] = r;
        }
    }
}

// The partial kernel, then the combine.  Store head_dims other than 64,
// 128 and 256 run on the padded kernels of the next of those geometries.
hipError_t launch_decode_attend(const AttendArgs& a, const AttendPlan& p, hipStream_t stream) {
    float* ws_o = static_cast<float*>(a.workspace);
    float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + p.ml_offset);
    const int ds = a.head_dim;
    if (ds < 16 || ds > 256 || ds % 16 != 0) return hipErrorInvalidValue;   // rejected by the ABI first
    const bool padded = ds != 64 && ds != 128 && ds != 256;
    hipError_t e;
    if (padded) e = launch_attend_partial_padded(a, p, ws_o, ws_ml, stream);
    else if (a.bf16) e = launch_attend_partial_bf16(a, p, ws_o, ws_ml, stream);
    else if (a.meta16) e = launch_partials<2, false>(a, p, ws_o, ws_ml, stream);
    else e = launch_partials<4, false>(a, p, ws_o, ws_ml, stream);
    if (e != hipSuccess) return e;
    const dim3 rows_grid(static_cast<uint32_t>(a.B * a.Hq));
    const bool many = p.n_split >= 48;
    const dim3 block(64 * (many ? 16 : 4));
    if (ds <= 64) {
        if (many) hipLaunchKernelGGL((attend_combine_kernel<16, 64>), rows_grid, block, 0, stream, ws_o, ws_ml, p.n_split, a.out, ds);
        else hipLaunchKernelGGL((attend_combine_kernel<4, 64>), rows_grid, block, 0, stream, ws_o, ws_ml, p.n_split, a.out, ds);
    } else if (ds > 128) {
        if (many) hipLaunchKernelGGL((attend_combine_kernel<16, 256>), rows_grid, block, 0, stream, ws_o, ws_ml, p.n_split, a.out, ds);
        else hipLaunchKernelGGL((attend_combine_kernel<4, 256>), rows_grid, block, 0, stream, ws_o, ws_ml, p.n_split, a.out, ds);
    } else {
        if (many) hipLaunchKernelGGL((attend_combine_kernel<16, 128>), rows_grid, block, 0, stream, ws_o, ws_ml, p.n_split, a.out, ds);
        else hipLaunchKernelGGL((attend_combine_kernel<4, 128>), rows_grid, block, 0, stream, ws_o, ws_ml, p.n_split, a.out, ds);
    }
    return hipGetLastError();
}

}  // namespace kivi
