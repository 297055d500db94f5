// attend.hip -- the decode attend for fp16 caches (the partial kernel of
// attend_device.h), the split plan, and the log-sum-exp combine kernel that
// both the fp16 and the bfloat16 attends finish with.
#include <algorithm>

#include "attend_device.h"

namespace kivi {

// Merge the splits of one (sequence, query head), base-2 log-sum-exp:
// o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i with M = max_i m_i.
// WAVES waves per row: wave w takes splits w, w + WAVES, ..., lane l
// channels 2l and 2l + 1 (lanes l < D/2); the waves' sums meet in LDS.  The
// first kU splits of every wave are loaded together with their (m, l)
// before the maximum is known, so a row of up to kU * WAVES splits costs one
// memory round trip; only longer rows loop over the rest.
template <int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void attend_combine_kernel(const float* __restrict__ ws_o,
                                                                   const float* __restrict__ ws_ml,
                                                                   int64_t n_part, float* __restrict__ out)
{
    constexpr int kU = 4;
    __shared__ float red_m[WAVES];
    __shared__ float red_l[WAVES];
    __shared__ float2 red_o[WAVES][64];
    const int64_t row = blockIdx.x;                  // b * Hq + h
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const float* ml = ws_ml + row * n_part * 2;
    const float2* o = reinterpret_cast<const float2*>(ws_o + row * n_part * D) + l;
    const bool has = l < D / 2;                      // the lane has channels (always at D = 128)

    float2 mv[kU], ov[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t i = w + static_cast<int64_t>(u) * WAVES;
        mv[u] = i < n_part ? *reinterpret_cast<const float2*>(ml + 2 * i) : make_float2(-INFINITY, 0.0f);
        ov[u] = (i < n_part && has) ? o[i * (D / 2)] : make_float2(0.0f, 0.0f);
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
    float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const float e = exp2f(mv[u].x - M);
        L = __builtin_fmaf(e, mv[u].y, L);
        acc.x = __builtin_fmaf(e, ov[u].x, acc.x);
        acc.y = __builtin_fmaf(e, ov[u].y, acc.y);
    }
    for (int64_t i = w + static_cast<int64_t>(kU) * WAVES; i < n_part; i += WAVES) {
        const float2 m2 = *reinterpret_cast<const float2*>(ml + 2 * i);
        const float2 o2 = has ? o[i * (D / 2)] : make_float2(0.0f, 0.0f);
        const float e = exp2f(m2.x - M);
        L = __builtin_fmaf(e, m2.y, L);
        acc.x = __builtin_fmaf(e, o2.x, acc.x);
        acc.y = __builtin_fmaf(e, o2.y, acc.y);
    }
    red_o[w][l] = acc;
    if (l == 0) red_l[w] = L;
    __syncthreads();
    if (w == 0) {
        float Lt = red_l[0];
        float2 at = red_o[0][l];
#pragma unroll
        for (int v = 1; v < WAVES; ++v) {
            Lt += red_l[v];
            at.x += red_o[v][l].x;
            at.y += red_o[v][l].y;
        }
        // a sequence with no tokens at all (only possible in a variable-length
        // batch) has every partial empty (m = -inf, l = 0): its output is zero
        const float2 r = Lt > 0.0f ? make_float2(at.x / Lt, at.y / Lt) : make_float2(0.0f, 0.0f);
        if (has) reinterpret_cast<float2*>(out + row * D)[l] = r;
    }
}

// Split of the token axis.  Small problems (no more 32-token steps than the
// chip holds waves) get one step per wave: everything is in flight at once.
// Larger ones get as few whole rounds of kWaveSlots waves as keep a wave at
// most kMaxStepsPerWave steps, with the steps spread evenly, so the last
// round is not a short tail.
AttendPlan plan_attend(int64_t B, int Hq, int Hkv, int64_t n_quant, int64_t n_res, bool varlen,
                       int head_dim, bool bf16) {
    const int64_t pairs = B * Hkv;
    const int64_t steps_q = (n_quant + kStep - 1) / kStep;
    const int64_t steps = steps_q + (n_res + kStep - 1) / kStep;
    const int64_t total = pairs * steps;
    const int64_t slots = bf16 ? kWaveSlotsBF16 : kWaveSlots;
    int64_t spw = 1;
    if (total > slots) {
        // A variable-length batch sizes the grid for its longest sequence;
        // the shorter ones leave waves with little or nothing to do, so it
        // gets four times finer splits and the hardware refills the freed
        // slots with the remaining work.
        const int64_t per_round = varlen ? slots * 4 : slots;
        const int64_t rounds = (total + per_round * kMaxStepsPerWave - 1) / (per_round * kMaxStepsPerWave);
        spw = (total + rounds * per_round - 1) / (rounds * per_round);
    }
    // Small and mid-size calls take fewer, longer waves: each wave pays a
    // fixed cost (query load, LDS setup, its partial and its share of the
    // combine), and about 700 waves with two steps of loads in flight each
    // already keep these sizes at their best.  Measured per call on MI355X
    // (steps per wave -> us): B=1 x 16384 tokens 2 -> 19.1, 6 -> 16.1;
    // B=4 x 2048: 1 -> 13.3, 3 -> 11.9; B=16 x 2048: 3 -> 23.0, 9 -> 19.9;
    // B=4 x 16384: 6 -> 31.2, 9 -> 30.3; B=32 x 2048: 6 -> 31.7, 9 -> 31.4.
    const int64_t longer = (total + 699) / 700;
    spw = std::max(spw, std::min<int64_t>(9, longer));
    // The generic kernel (head_dims other than 64 and 128) has no fixed cost
    // to amortize and is latency-bound per lane: one 64-token chunk per wave.
    if (head_dim != 64 && head_dim != 128) spw = std::min<int64_t>(spw, 2);
    AttendPlan p;
    p.steps_q = steps_q;
    p.steps_per_wave = spw;
    p.n_split = (steps + spw - 1) / spw;
    const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(Hq) * static_cast<size_t>(p.n_split);
    p.ml_offset = (rows * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    p.workspace_bytes = p.ml_offset + rows * 2 * sizeof(float);
    return p;
}

// The partial kernel, then the combine.
hipError_t launch_decode_attend(const AttendArgs& a, const AttendPlan& p, hipStream_t stream) {
    float* ws_o = static_cast<float*>(a.workspace);
    float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + p.ml_offset);
    if (a.head_dim != 64 && a.head_dim != 128) return launch_attend_generic(a, p, ws_o, ws_ml, stream);
    hipError_t e;
    if (a.bf16) e = launch_attend_partial_bf16(a, p, ws_o, ws_ml, stream);
    else if (a.meta16) e = launch_partials<2, false>(a, p, ws_o, ws_ml, stream);
    else e = launch_partials<4, false>(a, p, ws_o, ws_ml, stream);
    if (e != hipSuccess) return e;
    const dim3 rows_grid(static_cast<uint32_t>(a.B * a.Hq));
    const bool many = p.n_split >= 48;
    if (a.head_dim == 64) {
        if (many) hipLaunchKernelGGL((attend_combine_kernel<16, 64>), rows_grid, dim3(64 * 16), 0, stream, ws_o, ws_ml, p.n_split, a.out);
        else hipLaunchKernelGGL((attend_combine_kernel<4, 64>), rows_grid, dim3(64 * 4), 0, stream, ws_o, ws_ml, p.n_split, a.out);
    } else {
        if (many) hipLaunchKernelGGL((attend_combine_kernel<16, 128>), rows_grid, dim3(64 * 16), 0, stream, ws_o, ws_ml, p.n_split, a.out);
        else hipLaunchKernelGGL((attend_combine_kernel<4, 128>), rows_grid, dim3(64 * 4), 0, stream, ws_o, ws_ml, p.n_split, a.out);
    }
    return hipGetLastError();
}

}  // namespace kivi
