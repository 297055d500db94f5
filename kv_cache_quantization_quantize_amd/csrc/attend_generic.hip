// attend_generic.hip -- the decode attend at the head_dims the MFMA kernels
// of attend_device.h do not take: the multiples of 16 other than 64, 128
// and 256, with groups of 32 and binary32 scale/zero, for fp16 and bfloat16
// caches.
//
// Sources, cited by page title and section:
//   [Benchmarks] VeloxQuant-MLX "Benchmarks" page, "KV-Cache Kernel Roofline:
//                What Actually Limits Decode" (a decode+attend kernel reading
//                the packed state directly).
//   [Metal post] blog post "A 5.65x Metal Kernel That Made My LLM Exactly 0%
//                Faster", "Three ways to be off by one bit" (the
//                reconstruction rule the kernel rebuilds K and V with).
//
// A coverage path, not a tuned one: one 64-lane wave per (sequence, kv head,
// split of the token axis), the split plan and the partial (m, l, o) layout
// of the MFMA kernels.  Per 64-token chunk, lane = token computes the scores
// of every query head of the kv head over the exact 16-bit reconstruction of
// its key row; the online softmax runs in fp32 (base 2) across the wave;
// then lane = channel accumulates P V over the chunk's tokens, again from the
// exact reconstruction.  Nothing is rounded but the reconstruction itself.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

namespace {

constexpr int kMaxD = 256;
constexpr float kLog2eG = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// A stored 16-bit value, widened exactly.
template <bool BF>
__device__ __forceinline__ float widen16(uint16_t h) {
    if constexpr (BF) return __uint_as_float(static_cast<uint32_t>(h) << 16);
    else return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// The stored reconstruction of one element, widened: rne16(fl(fl(q s) + z)).
template <bool BF>
__device__ __forceinline__ float recon_value(uint32_t code, float s, float z) {
    const uint32_t bits = recon_out<BF>(static_cast<float>(code), s, z);
    return widen16<BF>(static_cast<uint16_t>(bits));
}

__device__ __forceinline__ int ring_at(int tok, int head, int ring) {
    const int r = tok + head;
    return r >= ring ? r - ring : r;
}

}  // namespace

// GQA (query heads per kv head) is a template parameter so that the
// per-head accumulators stay in registers under unrolled loops.
template <bool BF, int GQA>
__global__ __launch_bounds__(64) void attend_generic_kernel(const AttendArgs a, int spw, int steps_q,
                                                            int64_t n_split, float* __restrict__ ws_o,
                                                            float* __restrict__ ws_ml)
{
    constexpr int kG = 32;
    __shared__ float q_s[GQA][kMaxD];
    __shared__ float p_s[GQA][64];
    const int l = threadIdx.x;
    const int D = a.head_dim;
    const int bits = a.bits;
    const uint32_t mask = (1u << bits) - 1u;
    const int per_word = 32 / bits;
    const int W = D * bits / 32;                       // code words per token
    const int n_meta = (D + kG - 1) / kG;              // value groups per token
    const int split = blockIdx.x;
    const int64_t bkv = blockIdx.y;
    const int64_t b = bkv / a.Hkv;
    const int kv = static_cast<int>(bkv - b * a.Hkv);
    const int64_t qrow0 = b * a.Hq + static_cast<int64_t>(kv) * GQA;

    int nq = static_cast<int>(a.n_quant);
    int nr = static_cast<int>(a.n_res);
    if (a.seq_n_quant) {
        nq = min(max(a.seq_n_quant[b], 0), nq);
        nr = min(max(a.seq_n_res[b], 0), nr);
    }
    const int s0 = split * spw, s1 = s0 + spw;
    const int j0 = s0 * kG, j1 = min(min(s1, steps_q) * kG, nq);            // store tokens
    const int r0 = max(s0 - steps_q, 0) * kG, r1 = min(max(s1 - steps_q, 0) * kG, nr);   // residual

    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    for (int h = 0; h < GQA; ++h)
        for (int c = l; c < D; c += 64) q_s[h][c] = widen16<BF>(qp[(qrow0 + h) * D + c]);
    __syncthreads();

    const uint32_t* kc = a.k_codes + bkv * a.k_codes_bh_stride;
    const uint32_t* vc = a.v_codes + bkv * a.v_codes_bh_stride;
    const float* ksc = static_cast<const float*>(a.k_scale) + bkv * a.k_meta_bh_stride;
    const float* kze = static_cast<const float*>(a.k_zero) + bkv * a.k_meta_bh_stride;
    const float* vsc = static_cast<const float*>(a.v_scale) + bkv * a.v_meta_bh_stride;
    const float* vze = static_cast<const float*>(a.v_zero) + bkv * a.v_meta_bh_stride;
    const uint16_t* kr = a.k_res + bkv * a.res_bh_stride;
    const uint16_t* vr = a.v_res + bkv * a.res_bh_stride;
    const float c2 = a.softmax_scale * kLog2eG;

    float m[GQA], lsum[GQA], o[GQA][kMaxD / 64];
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.0f;
#pragma unroll
        for (int k = 0; k < kMaxD / 64; ++k) o[h][k] = 0.0f;
    }

    // two ranges: store tokens [j0, j1), then residual tokens [r0, r1)
    for (int part = 0; part < 2; ++part) {
        const bool store = part == 0;
        const int lo = store ? j0 : r0, hi = store ? j1 : r1;
        for (int t0 = lo; t0 < hi; t0 += 64) {           // wave-uniform
            // ---- scores: lane = token
            const int t = t0 + l;
            const bool live = t < hi;
            float s[GQA];
#pragma unroll
            for (int h = 0; h < GQA; ++h) s[h] = 0.0f;
            if (live) {
                if (store) {
                    const float* sp = ksc + static_cast<int64_t>(t / kG) * D;
                    const float* zp = kze + static_cast<int64_t>(t / kG) * D;
#pragma unroll 4
                    for (int w = 0; w < W; ++w) {
                        const uint32_t word = kc[static_cast<int64_t>(t) * W + w];
#pragma unroll 8
                        for (int j = 0; j < per_word; ++j) {
                            const int c = w * per_word + j;
                            const float kv_ = recon_value<BF>((word >> (bits * j)) & mask, sp[c], zp[c]);
#pragma unroll
                            for (int h = 0; h < GQA; ++h) s[h] = __builtin_fmaf(q_s[h][c], kv_, s[h]);
                        }
                    }
                } else {
                    const uint16_t* row = kr + static_cast<int64_t>(ring_at(t, a.res_head, a.res_ring)) * D;
#pragma unroll 8
                    for (int c = 0; c < D; ++c) {
                        const float kv_ = widen16<BF>(row[c]);
#pragma unroll
                        for (int h = 0; h < GQA; ++h) s[h] = __builtin_fmaf(q_s[h][c], kv_, s[h]);
                    }
                }
            }
            // ---- online softmax across the wave (the chunk has >= 1 live token)
#pragma unroll
            for (int h = 0; h < GQA; ++h) {
                const float sc = live ? s[h] * c2 : -INFINITY;
                const float m_new = fmaxf(m[h], wave_max(sc));
                const float alpha = exp2f(m[h] - m_new);    // m[h] = -inf on the first chunk: 0
                const float p = live ? exp2f(sc - m_new) : 0.0f;
                lsum[h] = lsum[h] * alpha + wave_sum(p);
#pragma unroll
                for (int k = 0; k < kMaxD / 64; ++k) o[h][k] *= alpha;
                m[h] = m_new;
                p_s[h][l] = p;
            }
            __syncthreads();
            // ---- P V: lane = channel
            const int n = min(64, hi - t0);
#pragma unroll
            for (int k = 0; k < kMaxD / 64; ++k) {
                const int c = l + 64 * k;
                if (c >= D) continue;
#pragma unroll 8
                for (int i = 0; i < n; ++i) {              // unrolled: several loads in flight
                    const int tt = t0 + i;
                    float v;
                    if (store) {
                        const uint32_t word = vc[static_cast<int64_t>(tt) * W + c / per_word];
                        const int64_t m_at = static_cast<int64_t>(tt) * n_meta + c / kG;
                        v = recon_value<BF>((word >> (bits * (c % per_word))) & mask, vsc[m_at], vze[m_at]);
                    } else {
                        v = widen16<BF>(vr[static_cast<int64_t>(ring_at(tt, a.res_head, a.res_ring)) * D + c]);
                    }
#pragma unroll
                    for (int h = 0; h < GQA; ++h) o[h][k] = __builtin_fmaf(p_s[h][i], v, o[h][k]);
                }
            }
            __syncthreads();
        }
    }

#pragma unroll
    for (int h = 0; h < GQA; ++h) {
        float* dst = ws_o + ((qrow0 + h) * n_split + split) * D;
#pragma unroll
        for (int k = 0; k < kMaxD / 64; ++k) {
            const int c = l + 64 * k;
            if (c < D) dst[c] = o[h][k];
        }
        if (l == 0) {
            float* ml = ws_ml + ((qrow0 + h) * n_split + split) * 2;
            ml[0] = m[h];
            ml[1] = lsum[h];
        }
    }
}

// Merge of the splits for any head_dim <= 256: lane l takes channels l,
// l + 64, ... (the MFMA kernels' combine takes channel pairs at 64, 128 and
// 256).
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void attend_combine_any_kernel(const float* __restrict__ ws_o,
                                                                       const float* __restrict__ ws_ml,
                                                                       int64_t n_split, float* __restrict__ out,
                                                                       int D)
{
    __shared__ float red_m[WAVES];
    __shared__ float red_l[WAVES];
    __shared__ float red_o[WAVES][kMaxD];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const float* ml = ws_ml + row * n_split * 2;
    const float* o = ws_o + row * n_split * D;
    float M = -INFINITY;
    for (int64_t i = t; i < n_split; i += 64 * WAVES) M = fmaxf(M, ml[2 * i]);
    M = wave_max(M);
    if (l == 0) red_m[w] = M;
    __syncthreads();
    M = red_m[0];
    for (int i = 1; i < WAVES; ++i) M = fmaxf(M, red_m[i]);
    if (M == -INFINITY) M = 0.0f;                    // every split empty
    float L = 0.0f;
    float acc[kMaxD / 64];
#pragma unroll
    for (int k = 0; k < kMaxD / 64; ++k) acc[k] = 0.0f;
    for (int64_t i = w; i < n_split; i += WAVES) {
        const float e = exp2f(ml[2 * i] - M);
        L = __builtin_fmaf(e, ml[2 * i + 1], L);
#pragma unroll
        for (int k = 0; k < kMaxD / 64; ++k) {
            const int c = l + 64 * k;
            if (c < D) acc[k] = __builtin_fmaf(e, o[i * D + c], acc[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxD / 64; ++k) {
        const int c = l + 64 * k;
        if (c < D) red_o[w][c] = acc[k];
    }
    if (l == 0) red_l[w] = L;
    __syncthreads();
    if (w == 0) {
        float Lt = red_l[0];
        for (int v = 1; v < WAVES; ++v) Lt += red_l[v];
#pragma unroll
        for (int k = 0; k < kMaxD / 64; ++k) {
            const int c = l + 64 * k;
            if (c >= D) continue;
            float at = red_o[0][c];
            for (int v = 1; v < WAVES; ++v) at += red_o[v][c];
            out[row * D + c] = Lt > 0.0f ? at / Lt : 0.0f;
        }
    }
}

hipError_t launch_attend_generic(const AttendArgs& a, const AttendPlan& p, float* ws_o, float* ws_ml,
                                 hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(p.n_split), static_cast<uint32_t>(a.B * a.Hkv));
    const int spw = static_cast<int>(p.steps_per_wave), sq = static_cast<int>(p.steps_q);
#define KIVI_GENERIC(BFV, G) hipLaunchKernelGGL((attend_generic_kernel<BFV, G>), grid, dim3(64), 0, stream, a, spw, sq, p.n_split, ws_o, ws_ml)
    switch ((a.Hq / a.Hkv) * 2 + (a.bf16 ? 1 : 0)) {
        case 2: KIVI_GENERIC(false, 1); break;
        case 3: KIVI_GENERIC(true, 1); break;
        case 4: KIVI_GENERIC(false, 2); break;
        case 5: KIVI_GENERIC(true, 2); break;
        case 8: KIVI_GENERIC(false, 4); break;
        case 9: KIVI_GENERIC(true, 4); break;
        case 16: KIVI_GENERIC(false, 8); break;
        default: KIVI_GENERIC(true, 8); break;          // 17: the ABI admits only 1, 2, 4 and 8
    }
#undef KIVI_GENERIC
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 rows(static_cast<uint32_t>(a.B * a.Hq));
    if (p.n_split >= 48)
        hipLaunchKernelGGL(attend_combine_any_kernel<16>, rows, dim3(64 * 16), 0, stream, ws_o, ws_ml, p.n_split, a.out, a.head_dim);
    else
        hipLaunchKernelGGL(attend_combine_any_kernel<4>, rows, dim3(64 * 4), 0, stream, ws_o, ws_ml, p.n_split, a.out, a.head_dim);
    return hipGetLastError();
}

}  // namespace kivi
