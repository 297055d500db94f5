// attend.hip -- fused dequantize + attend for one new query token per
// sequence over a packed 2/4-bit store plus an fp16 residual window.
//
// Sources, cited by page title and section:
//   [Benchmarks] VeloxQuant-MLX "Benchmarks" page, "KV-Cache Kernel Roofline:
//                What Actually Limits Decode": the Metal decode+attend kernel
//                ran one threadgroup per (batch, head) and was bound by how
//                few threadgroups that dispatches (8 at B=1, H=8), not by
//                bandwidth; head-packing K/V across query heads cut the
//                threadgroup count further and lost.
//   [Metal post] blog post "A 5.65x Metal Kernel That Made My LLM Exactly 0%
//                Faster", "What we're actually optimizing" (the newest tokens
//                stay fp16) and "So why does the kernel ship?" (dequantize
//                in registers inside attention).
//
// Design for MI355X: one workgroup per (sequence, kv head, token split).  The
// workgroup serves every query head that shares the kv head, so each packed
// byte is read from HBM once; the token axis is split so the grid reaches
// thousands of workgroups even at B=1 (which answers the occupancy limit the
// pages measured).  Partials (m, l, o[128]) go to the workspace and a second
// kernel merges them with the log-sum-exp rule.
//
// Arithmetic: scores and the weighted sum accumulate in fp32; K and V are the
// exact fp16 reconstructions of the store (the same values kivi_dequantize
// writes).
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

constexpr int kMaxChunk = 256;

template <int BITS>
__device__ __forceinline__ void load_key8(const uint32_t* __restrict__ codes, const float* __restrict__ sc,
                                          const float* __restrict__ ze, int64_t j, int c, float (&kf)[8]) {
    constexpr int kWords = kHeadDim * BITS / 32;
    constexpr uint32_t kMask = (1u << BITS) - 1u;
    uint32_t w;
    if constexpr (BITS == 4) w = codes[j * kWords + c];
    else w = codes[j * kWords + (c >> 1)] >> (16 * (c & 1));
    const float* sp = sc + (j / kGroup) * kHeadDim + c * 8;
    const float* zp = ze + (j / kGroup) * kHeadDim + c * 8;
    const float4 s0 = *reinterpret_cast<const float4*>(sp);
    const float4 s1 = *reinterpret_cast<const float4*>(sp + 4);
    const float4 z0 = *reinterpret_cast<const float4*>(zp);
    const float4 z1 = *reinterpret_cast<const float4*>(zp + 4);
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const float z[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) kf[k] = f16_to_f32(recon_f16((w >> (BITS * k)) & kMask, s[k], z[k]));
}

template <int BITS>
__device__ __forceinline__ void load_value8(const uint32_t* __restrict__ codes, const float* __restrict__ sc,
                                            const float* __restrict__ ze, int64_t j, int c, float (&vf)[8]) {
    constexpr int kWords = kHeadDim * BITS / 32;
    constexpr uint32_t kMask = (1u << BITS) - 1u;
    constexpr int kMetaPerTok = kHeadDim / kGroup;
    uint32_t w;
    if constexpr (BITS == 4) w = codes[j * kWords + c];
    else w = codes[j * kWords + (c >> 1)] >> (16 * (c & 1));
    const float s = sc[j * kMetaPerTok + (c >> 2)];
    const float z = ze[j * kMetaPerTok + (c >> 2)];
#pragma unroll
    for (int k = 0; k < 8; ++k) vf[k] = f16_to_f32(recon_f16((w >> (BITS * k)) & kMask, s, z));
}

template <int BITS, int GQA>
__global__ __launch_bounds__(kBlock) void attend_partial_kernel(const AttendArgs a, int64_t chunk,
                                                                int64_t n_split, float* __restrict__ ws_o,
                                                                float* __restrict__ ws_ml)
{
    __shared__ float q_s[GQA][kHeadDim];
    __shared__ float p_s[GQA][kMaxChunk];
    __shared__ float red[kWavesPerBlock][GQA][kHeadDim];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t split = blockIdx.x;
    const int64_t bkv = blockIdx.y;                  // b * Hkv + kv
    const int64_t b = bkv / a.Hkv;
    const int kv = static_cast<int>(bkv - b * a.Hkv);
    const int64_t N = a.n_quant + a.n_res;
    const int64_t j0 = split * chunk;
    const int n_tok = static_cast<int>((j0 + chunk < N ? j0 + chunk : N) - j0);
    const int64_t qrow0 = b * a.Hq + static_cast<int64_t>(kv) * GQA;

    for (int idx = tid; idx < GQA * kHeadDim; idx += kBlock)
        q_s[idx / kHeadDim][idx % kHeadDim] = f16_to_f32(a.q[qrow0 * kHeadDim + idx]);
    __syncthreads();

    const int c = tid & 15;                          // channels 8c .. 8c+7
    const int row = tid >> 4;                        // 16 token rows per pass
    const uint32_t* kc = a.k_codes + bkv * a.k_codes_bh_stride;
    const float* ks = a.k_scale + bkv * a.k_meta_bh_stride;
    const float* kz = a.k_zero + bkv * a.k_meta_bh_stride;
    const uint32_t* vc = a.v_codes + bkv * a.v_codes_bh_stride;
    const float* vs = a.v_scale + bkv * a.v_meta_bh_stride;
    const float* vz = a.v_zero + bkv * a.v_meta_bh_stride;
    const uint16_t* kr = a.k_res + bkv * a.res_bh_stride;
    const uint16_t* vr = a.v_res + bkv * a.res_bh_stride;

    // ---- scores s[h][t] = (q_h . k_t) * softmax_scale
    float qreg[GQA][8];
#pragma unroll
    for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int k = 0; k < 8; ++k) qreg[h][k] = q_s[h][c * 8 + k];

    for (int t0 = 0; t0 < n_tok; t0 += 16) {         // uniform trip count
        const int t = t0 + row;
        const bool valid = t < n_tok;
        const int64_t j = j0 + (valid ? t : 0);
        float kf[8];
        if (j < a.n_quant) {
            load_key8<BITS>(kc, ks, kz, j, c, kf);
        } else {
            const uint4 v = *reinterpret_cast<const uint4*>(kr + (j - a.n_quant) * kHeadDim + c * 8);
            unpack8(v, kf);
        }
        float part[GQA];
#pragma unroll
        for (int h = 0; h < GQA; ++h) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc = __builtin_fmaf(qreg[h][k], kf[k], acc);
            acc += __shfl_xor(acc, 1);
            acc += __shfl_xor(acc, 2);
            acc += __shfl_xor(acc, 4);
            acc += __shfl_xor(acc, 8);
            part[h] = acc;
        }
        if (valid && c == 0) {
#pragma unroll
            for (int h = 0; h < GQA; ++h) p_s[h][t] = part[h] * a.softmax_scale;
        }
    }
    __syncthreads();

    // ---- softmax over the split: wave w owns heads w, w+4, ...
    for (int h = wave; h < GQA; h += kWavesPerBlock) {
        float m = -INFINITY;
        for (int t = lane; t < n_tok; t += 64) m = fmaxf(m, p_s[h][t]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        float l = 0.0f;
        for (int t = lane; t < n_tok; t += 64) {
            const float p = __expf(p_s[h][t] - m);
            p_s[h][t] = p;
            l += p;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
        if (lane == 0) {
            float* ml = ws_ml + ((qrow0 + h) * n_split + split) * 2;
            ml[0] = m;
            ml[1] = l;
        }
    }
    __syncthreads();

    // ---- o[h][d] = sum_t p[h][t] * v[t][d]
    float acc[GQA][8];
#pragma unroll
    for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = 0.0f;

    for (int t0 = 0; t0 < n_tok; t0 += 16) {
        const int t = t0 + row;
        const bool valid = t < n_tok;
        const int64_t j = j0 + (valid ? t : 0);
        float vf[8];
        if (j < a.n_quant) {
            load_value8<BITS>(vc, vs, vz, j, c, vf);
        } else {
            const uint4 v = *reinterpret_cast<const uint4*>(vr + (j - a.n_quant) * kHeadDim + c * 8);
            unpack8(v, vf);
        }
#pragma unroll
        for (int h = 0; h < GQA; ++h) {
            const float p = valid ? p_s[h][t] : 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[h][k] = __builtin_fmaf(p, vf[k], acc[h][k]);
        }
    }
    // rows 4w .. 4w+3 of wave w meet in lanes 0..15
#pragma unroll
    for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            acc[h][k] += __shfl_xor(acc[h][k], 16);
            acc[h][k] += __shfl_xor(acc[h][k], 32);
        }
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < GQA; ++h)
#pragma unroll
            for (int k = 0; k < 8; ++k) red[wave][h][c * 8 + k] = acc[h][k];
    }
    __syncthreads();
    for (int idx = tid; idx < GQA * kHeadDim; idx += kBlock) {
        const int h = idx / kHeadDim;
        const int d = idx % kHeadDim;
        const float o = (red[0][h][d] + red[1][h][d]) + (red[2][h][d] + red[3][h][d]);
        ws_o[((qrow0 + h) * n_split + split) * kHeadDim + d] = o;
    }
}

// Merge the splits of one (sequence, query head): o = sum_i e^(m_i - M) o_i /
// sum_i e^(m_i - M) l_i with M = max_i m_i.
__global__ __launch_bounds__(kHeadDim) void attend_combine_kernel(const float* __restrict__ ws_o,
                                                                  const float* __restrict__ ws_ml,
                                                                  int64_t n_split, float* __restrict__ out)
{
    const int64_t row = blockIdx.x;                  // b * Hq + h
    const int d = threadIdx.x;
    const float* ml = ws_ml + row * n_split * 2;
    float M = -INFINITY;
    for (int64_t i = 0; i < n_split; ++i) M = fmaxf(M, ml[2 * i]);
    float L = 0.0f, acc = 0.0f;
    for (int64_t i = 0; i < n_split; ++i) {
        const float w = __expf(ml[2 * i] - M);
        L = __builtin_fmaf(w, ml[2 * i + 1], L);
        acc = __builtin_fmaf(w, ws_o[(row * n_split + i) * kHeadDim + d], acc);
    }
    out[row * kHeadDim + d] = acc / L;
}

AttendPlan plan_attend(int64_t B, int Hq, int Hkv, int64_t n_quant, int64_t n_res) {
    (void)Hq;
    const int64_t N = n_quant + n_res;
    const int64_t pairs = B * Hkv;
    int64_t chunk = kMaxChunk;
    // smaller splits until the grid holds >= 4 workgroups per CU (256 CUs)
    while (chunk > 32 && pairs * ((N + chunk - 1) / chunk) < 1024) chunk /= 2;
    AttendPlan p;
    p.chunk = chunk;
    p.n_split = (N + chunk - 1) / chunk;
    const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(Hq) * static_cast<size_t>(p.n_split);
    const size_t o_bytes = (rows * kHeadDim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    p.workspace_bytes = o_bytes + rows * 2 * sizeof(float);
    return p;
}

template <int BITS, int GQA>
static hipError_t launch_t(const AttendArgs& a, const AttendPlan& p, hipStream_t stream) {
    float* ws_o = static_cast<float*>(a.workspace);
    const size_t rows = static_cast<size_t>(a.B) * a.Hq * p.n_split;
    const size_t o_bytes = (rows * kHeadDim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + o_bytes);
    const dim3 grid(static_cast<uint32_t>(p.n_split), static_cast<uint32_t>(a.B * a.Hkv));
    hipLaunchKernelGGL((attend_partial_kernel<BITS, GQA>), grid, dim3(kBlock), 0, stream, a,
                       p.chunk, p.n_split, ws_o, ws_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_combine_kernel, dim3(static_cast<uint32_t>(a.B * a.Hq)),
                       dim3(kHeadDim), 0, stream, ws_o, ws_ml, p.n_split, a.out);
    return hipGetLastError();
}

template <int BITS>
static hipError_t launch_bits(const AttendArgs& a, const AttendPlan& p, hipStream_t stream) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_t<BITS, 1>(a, p, stream);
        case 2: return launch_t<BITS, 2>(a, p, stream);
        case 4: return launch_t<BITS, 4>(a, p, stream);
        default: return launch_t<BITS, 8>(a, p, stream);
    }
}

hipError_t launch_decode_attend(const AttendArgs& a, const AttendPlan& p, hipStream_t stream) {
    return a.bits == 4 ? launch_bits<4>(a, p, stream) : launch_bits<2>(a, p, stream);
}

}  // namespace kivi
