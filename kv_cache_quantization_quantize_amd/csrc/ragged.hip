// ragged.hip -- flush and dequantize for the head_dims the tiled kernels of
// flush.hip and dequant.hip do not cover: every multiple of 16 from 16 to
// 256 other than 64, 128 and 256 (80, 96 and 112 among them), with groups of
// 32.  When 32 does not divide head_dim, a token's last value group is the
// remaining 16 channels.
//
// Sources, cited by page title and section:
//   [Metal post] blog post "A 5.65x Metal Kernel That Made My LLM Exactly 0%
//                Faster": "What we're actually optimizing" (the quantizer),
//                "Kernel B" (a token's channel groups, the last one ragged),
//                "Three ways to be off by one bit" (ties to even, two
//                roundings in the reconstruction, edge padding of a ragged
//                token group).
//
// One wave per 32-token x head_dim tile.  A token row is nC = head_dim/8
// chunks of 8 channels (16 B); lane = r * nC + c takes chunk c of rows
// r, r + nR, ... with nR = 64 / nC row phases (lanes past nR * nC only take
// part in the exchanges).  Partial min/max meet in the wave's own LDS
// region.  The arithmetic is that of the tiled kernels (kivi_device.h): the
// scale shortcut, the reciprocal code with its near-tie fallback to the IEEE
// quotient, and the bfloat16 guards; their proofs are per group and per
// element, so they hold at any head_dim.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

namespace {

constexpr int kG = 32;
constexpr int kMaxD = 256;
// rows per lane: 32 / (64 / (head_dim / 8)) rounded up, at most 16 (head_dim
// 256 has two row phases); loops run to this bound under a wave-uniform
// guard, so a lane issues all its loads before it waits on the first
constexpr int kMaxIters = 16;

// The wave's LDS: per-phase min/max of every channel (keys) or per-row
// min/max of every chunk (values), then the tile's scale and zero.
struct RaggedSmem {
    float mn[kG][kMaxD / 8 > kG ? kMaxD / 8 : kG];
    float mx[kG][kMaxD / 8 > kG ? kMaxD / 8 : kG];
};
struct KeySmem {
    float mn[512];          // [phase][channel], phases * head_dim <= 512
    float mx[512];
    float sc[kMaxD];
    float ze[kMaxD];
};

// Keeps the compiler from moving LDS accesses across this point.  Each wave
// uses its own LDS region and a wave's LDS instructions execute in order, so
// no hardware barrier is needed between one lane's write and another's read.
__device__ __forceinline__ void lds_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

__device__ __forceinline__ float widen(const uint4& raw, int j, bool bf16) {
    const uint32_t w = word_of(raw, j >> 1);
    if (bf16) return (j & 1) ? bf16_hi(w) : bf16_lo(w);
    return static_cast<float>(as_h2(w)[j & 1]);
}

}  // namespace

// Keys: one wave per (slab, token group of 32).
template <int BITS, bool RECON, bool BF16>
__global__ __launch_bounds__(kBlock) void key_flush_ragged_kernel(
    const uint16_t* __restrict__ x, int64_t S, int64_t x_bh_stride,
    uint32_t* __restrict__ codes, int64_t codes_bh_stride,
    float* __restrict__ scale, float* __restrict__ zero, int64_t meta_bh_stride,
    int64_t dst_token, uint16_t* __restrict__ recon, int64_t recon_bh_stride,
    int64_t n_groups, int64_t n_tiles, int D, float one)
{
    __shared__ KeySmem smem[kWavesPerBlock];
    constexpr float kL = static_cast<float>((1 << BITS) - 1);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
    if (tile >= n_tiles) return;                       // uniform across the wave
    KeySmem& sm = smem[wave];
    const int nC = D / 8, nR = 64 / nC;
    const int c = lane % nC, r = lane / nC;
    const bool on = r < nR;
    const int kWords = D * BITS / 32;
    const int64_t bh = tile / n_groups;
    const int64_t g = tile - bh * n_groups;
    const int64_t s0 = g * kG;
    const int n_rows = static_cast<int>(S - s0 < kG ? S - s0 : kG);
    const uint16_t* xt = x + bh * x_bh_stride + s0 * D;
    const int iters = (kG + nR - 1) / nR;

    // per-lane min/max over its rows; a row past the group's real rows (or
    // past 32) re-reads the last real row, which cannot move min or max
    uint4 raw[kMaxIters];
#pragma unroll
    for (int i = 0; i < kMaxIters; ++i) {
        const int row = r + nR * i;
        if (i < iters) raw[i] = load_stream(xt + (row < n_rows ? row : n_rows - 1) * D + c * 8);
    }
    float mn[8], mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { mn[j] = widen(raw[0], j, BF16); mx[j] = mn[j]; }
#pragma unroll
    for (int i = 1; i < kMaxIters; ++i) {
        if (i >= iters) continue;                   // wave-uniform
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = widen(raw[i], j, BF16);
            mn[j] = fminimum(mn[j], v);
            mx[j] = fmaximum(mx[j], v);
        }
    }
    lds_fence();
    if (on) {
#pragma unroll
        for (int j = 0; j < 8; ++j) { sm.mn[r * D + c * 8 + j] = mn[j]; sm.mx[r * D + c * 8 + j] = mx[j]; }
    }
    lds_fence();
    // phase 0 finishes its chunk: zero = min, scale = RN((max - min) / L)
    if (on && r == 0) {
        float sc[8], ze[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float a = mn[j], b = mx[j];
            for (int p = 1; p < nR; ++p) {
                a = fminimum(a, sm.mn[p * D + c * 8 + j]);
                b = fmaximum(b, sm.mx[p * D + c * 8 + j]);
            }
            ze[j] = canon_zero(a);
            sc[j] = BF16 ? scale_wide<BITS>(b - a) : scale_of<BITS>(b - a);
            sm.sc[c * 8 + j] = sc[j];
            sm.ze[c * 8 + j] = ze[j];
        }
        const int64_t moff = bh * meta_bh_stride + (dst_token / kG + g) * D + c * 8;
        store_stream4(scale + moff, sc[0], sc[1], sc[2], sc[3]);
        store_stream4(scale + moff + 4, sc[4], sc[5], sc[6], sc[7]);
        store_stream4(zero + moff, ze[0], ze[1], ze[2], ze[3]);
        store_stream4(zero + moff + 4, ze[4], ze[5], ze[6], ze[7]);
    }
    lds_fence();
    float sc[8], ze[8], rc[8];
    bool slow = false;                                 // a bfloat16 scale off the fast path
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sc[j] = sm.sc[c * 8 + j];
        ze[j] = sm.ze[c * 8 + j];
        rc[j] = recip_clamped(sc[j]);
        if constexpr (BF16) slow |= !fast_scale(sc[j]);
    }

    uint32_t* ct = codes + bh * codes_bh_stride + (dst_token + s0) * kWords;
    uint16_t* rt = RECON ? recon + bh * recon_bh_stride + s0 * D : nullptr;
#pragma unroll
    for (int i = 0; i < kMaxIters; ++i) {               // the same trip count on every lane
        if (i >= iters) continue;                   // wave-uniform
        const int row = r + nR * i;
        const bool live = on && row < n_rows;
        float t[8], qf[8];
        float dev = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            t[j] = sub_elem<BF16>(raw[i], j, one, ze[j]);
            qf[j] = quant_fast(t[j], rc[j], dev);
        }
        if (dev > kNearTie || slow) {                   // rare: within 2^-16 of a tie
#pragma unroll
            for (int j = 0; j < 8; ++j) qf[j] = quant_exact(t[j], sc[j], kL);
        }
        uint32_t packed = static_cast<uint32_t>(qf[0]);
#pragma unroll
        for (int j = 1; j < 8; ++j) packed |= static_cast<uint32_t>(qf[j]) << (BITS * j);
        if constexpr (BITS == 4) {
            if (live) store_stream(&ct[row * kWords + c], packed);
        } else {
            // 16 channels per word: the even chunk takes its odd neighbour's half
            const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(packed), 1));
            if (live && (c & 1) == 0) store_stream(&ct[row * kWords + (c >> 1)], packed | (hi << 16));
        }
        if constexpr (RECON) {
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = recon_out<BF16>(qf[j], sc[j], ze[j]);
            if (live) store_stream(rt + row * D + c * 8, pack8(h));
        }
    }
}

// Values: one wave per (slab, 32-token tile); a token's groups are chunks
// 4j .. 4j+3 (the last group of a head_dim that 32 does not divide has 2).
// QUAD (head_dim a multiple of 32): a row is a whole number of quads, so a
// group's four chunks are the four lanes of one DPP quad and its min and max
// meet in two quad exchanges instead of LDS.
template <int BITS, bool RECON, bool BF16, bool QUAD>
__global__ __launch_bounds__(kBlock) void value_flush_ragged_kernel(
    const uint16_t* __restrict__ x, int64_t S, int64_t x_bh_stride,
    uint32_t* __restrict__ codes, int64_t codes_bh_stride,
    float* __restrict__ scale, float* __restrict__ zero, int64_t meta_bh_stride,
    int64_t dst_token, uint16_t* __restrict__ recon, int64_t recon_bh_stride,
    int64_t tiles_per_bh, int64_t n_tiles, int D, float one)
{
    __shared__ RaggedSmem smem[kWavesPerBlock];
    constexpr float kL = static_cast<float>((1 << BITS) - 1);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
    if (tile >= n_tiles) return;                       // uniform across the wave
    RaggedSmem& sm = smem[wave];
    const int nC = D / 8, nR = 64 / nC;
    const int c = lane % nC, r = lane / nC;
    const bool on = r < nR;
    const int kWords = D * BITS / 32;
    const int n_meta = (D + kG - 1) / kG;              // groups per token
    const int j = c / 4;                               // the lane's group
    const int c_end = (4 * j + 4 < nC) ? 4 * j + 4 : nC;
    const int64_t bh = tile / tiles_per_bh;
    const int64_t s0 = (tile - bh * tiles_per_bh) * kG;
    const int n_rows = static_cast<int>(S - s0 < kG ? S - s0 : kG);
    const uint16_t* xt = x + bh * x_bh_stride + s0 * D;
    const int iters = (kG + nR - 1) / nR;

    // every row's chunk min/max into LDS (rows past the tile re-read row 0
    // and are never used); QUAD reduces each row in the loop below instead
    uint4 raw[kMaxIters];
#pragma unroll
    for (int i = 0; i < kMaxIters; ++i) {
        const int row = r + nR * i;
        if (i < iters) raw[i] = load_stream(xt + (on && row < n_rows ? row : 0) * D + c * 8);
    }
    if constexpr (!QUAD) {
#pragma unroll
        for (int i = 0; i < kMaxIters; ++i) {
            if (i >= iters) continue;               // wave-uniform
            const int row = r + nR * i;
            if (on && row < n_rows) {
                float a = widen(raw[i], 0, BF16), b = a;
#pragma unroll
                for (int k = 1; k < 8; ++k) {
                    const float v = widen(raw[i], k, BF16);
                    a = fminimum(a, v);
                    b = fmaximum(b, v);
                }
                sm.mn[row][c] = a;
                sm.mx[row][c] = b;
            }
        }
        lds_fence();
    }
    uint32_t* ct = codes + bh * codes_bh_stride + (dst_token + s0) * kWords;
    uint16_t* rt = RECON ? recon + bh * recon_bh_stride + s0 * D : nullptr;
#pragma unroll
    for (int i = 0; i < kMaxIters; ++i) {               // the same trip count on every lane
        if (i >= iters) continue;                   // wave-uniform
        const int row = r + nR * i;
        const bool live = on && row < n_rows;
        float lo = 0.0f, hi = 0.0f;
        if constexpr (QUAD) {
            // every lane takes part in the exchanges (idle lanes form their
            // own quads, rows past the tile hold row 0; neither is stored)
            lo = widen(raw[i], 0, BF16);
            hi = lo;
#pragma unroll
            for (int k = 1; k < 8; ++k) {
                const float v = widen(raw[i], k, BF16);
                lo = fminimum(lo, v);
                hi = fmaximum(hi, v);
            }
            lo = fminimum(lo, __uint_as_float(quad_xor1(__float_as_uint(lo))));
            hi = fmaximum(hi, __uint_as_float(quad_xor1(__float_as_uint(hi))));
            lo = fminimum(lo, __uint_as_float(quad_xor2(__float_as_uint(lo))));
            hi = fmaximum(hi, __uint_as_float(quad_xor2(__float_as_uint(hi))));
            if (!live) lo = hi = 0.0f;
        } else if (live) {
            lo = sm.mn[row][4 * j];
            hi = sm.mx[row][4 * j];
            for (int k = 4 * j + 1; k < c_end; ++k) {
                lo = fminimum(lo, sm.mn[row][k]);
                hi = fmaximum(hi, sm.mx[row][k]);
            }
        }
        const float ze = canon_zero(lo);
        const float sc = BF16 ? scale_wide<BITS>(hi - lo) : scale_of<BITS>(hi - lo);
        const float rc = recip_clamped(sc);
        float t[8], qf[8];
        float dev = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            t[k] = sub_elem<BF16>(raw[i], k, one, ze);
            qf[k] = quant_fast(t[k], rc, dev);
        }
        if (dev > kNearTie || (BF16 && !fast_scale(sc))) {
#pragma unroll
            for (int k = 0; k < 8; ++k) qf[k] = quant_exact(t[k], sc, kL);
        }
        uint32_t packed = static_cast<uint32_t>(qf[0]);
#pragma unroll
        for (int k = 1; k < 8; ++k) packed |= static_cast<uint32_t>(qf[k]) << (BITS * k);
        if constexpr (BITS == 4) {
            if (live) store_stream(&ct[row * kWords + c], packed);
        } else {
            const uint32_t hw = static_cast<uint32_t>(__shfl_xor(static_cast<int>(packed), 1));
            if (live && (c & 1) == 0) store_stream(&ct[row * kWords + (c >> 1)], packed | (hw << 16));
        }
        if (live) {
            const int64_t m = bh * meta_bh_stride + (dst_token + s0 + row) * n_meta + j;
            if (c % 4 == 0) scale[m] = sc;
            else if (c % 4 == 1) zero[m] = ze;
        }
        if constexpr (RECON) {
            uint32_t h[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) h[k] = recon_out<BF16>(qf[k], sc, ze);
            if (live) store_stream(rt + row * D + c * 8, pack8(h));
        }
    }
}

// Dequantize: one wave per (slab, 32 output rows).
template <int BITS, bool KEYS, bool BF16>
__global__ __launch_bounds__(kBlock) void dequant_ragged_kernel(
    const uint32_t* __restrict__ codes, int64_t codes_bh_stride,
    const float* __restrict__ scale, const float* __restrict__ zero, int64_t meta_bh_stride,
    int64_t t0, int64_t n, uint16_t* __restrict__ out, int64_t out_bh_stride,
    int64_t tiles_per_bh, int64_t n_tiles, int D)
{
    constexpr uint32_t kMask = (1u << BITS) - 1u;
    const int lane = threadIdx.x & 63;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;
    const int nC = D / 8, nR = 64 / nC;
    const int c = lane % nC, r = lane / nC;
    if (r >= nR) return;                               // no exchanges below
    const int kWords = D * BITS / 32;
    const int n_meta = (D + kG - 1) / kG;
    const int64_t bh = tile / tiles_per_bh;
    const int64_t i0 = (tile - bh * tiles_per_bh) * kG;
    const int64_t rows = n - i0 < kG ? n - i0 : kG;
    const uint32_t* cb = codes + bh * codes_bh_stride;
    const float* scb = scale + bh * meta_bh_stride;
    const float* zeb = zero + bh * meta_bh_stride;
    for (int k = r; k < rows; k += nR) {
        const int64_t t = t0 + i0 + k;
        uint32_t w;
        if constexpr (BITS == 4) w = cb[t * kWords + c];
        else w = cb[t * kWords + (c >> 1)] >> (16 * (c & 1));
        float sc[8], ze[8];
        if constexpr (KEYS) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sc[j] = scb[(t / kG) * D + c * 8 + j];
                ze[j] = zeb[(t / kG) * D + c * 8 + j];
            }
        } else {
            const float s = scb[t * n_meta + c / 4], z = zeb[t * n_meta + c / 4];
#pragma unroll
            for (int j = 0; j < 8; ++j) { sc[j] = s; ze[j] = z; }
        }
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = recon_out<BF16>(static_cast<float>((w >> (BITS * j)) & kMask), sc[j], ze[j]);
        store_stream(out + bh * out_bh_stride + (i0 + k) * D + c * 8, pack8(h));
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <bool KEYS, int BITS, bool RECON, bool BF16>
static hipError_t launch_flush_ragged_t(const FlushArgs& a, hipStream_t stream) {
    const int64_t per_bh = (a.S + kG - 1) / kG;
    const int64_t n_tiles = a.BH * per_bh;
    const int64_t blocks = (n_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    float* sc = static_cast<float*>(a.scale);
    float* ze = static_cast<float*>(a.zero);
    if constexpr (KEYS)
        hipLaunchKernelGGL((key_flush_ragged_kernel<BITS, RECON, BF16>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kBlock), 0, stream, a.x, a.S, a.x_bh_stride, a.codes, a.codes_bh_stride,
                           sc, ze, a.meta_bh_stride, a.dst_token, a.recon, a.recon_bh_stride,
                           per_bh, n_tiles, a.head_dim, 1.0f);
    else if (a.head_dim % kG == 0)
        hipLaunchKernelGGL((value_flush_ragged_kernel<BITS, RECON, BF16, true>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kBlock), 0, stream, a.x, a.S, a.x_bh_stride, a.codes, a.codes_bh_stride,
                           sc, ze, a.meta_bh_stride, a.dst_token, a.recon, a.recon_bh_stride,
                           per_bh, n_tiles, a.head_dim, 1.0f);
    else
        hipLaunchKernelGGL((value_flush_ragged_kernel<BITS, RECON, BF16, false>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kBlock), 0, stream, a.x, a.S, a.x_bh_stride, a.codes, a.codes_bh_stride,
                           sc, ze, a.meta_bh_stride, a.dst_token, a.recon, a.recon_bh_stride,
                           per_bh, n_tiles, a.head_dim, 1.0f);
    return hipGetLastError();
}

template <bool KEYS, bool BF16>
static hipError_t launch_flush_ragged_fmt(const FlushArgs& a, hipStream_t stream) {
    const bool rec = a.recon != nullptr;
    if (a.bits == 4) return rec ? launch_flush_ragged_t<KEYS, 4, true, BF16>(a, stream)
                                : launch_flush_ragged_t<KEYS, 4, false, BF16>(a, stream);
    return rec ? launch_flush_ragged_t<KEYS, 2, true, BF16>(a, stream)
               : launch_flush_ragged_t<KEYS, 2, false, BF16>(a, stream);
}

hipError_t launch_flush_ragged(bool keys, const FlushArgs& a, hipStream_t stream) {
    if (keys) return a.bf16 ? launch_flush_ragged_fmt<true, true>(a, stream) : launch_flush_ragged_fmt<true, false>(a, stream);
    return a.bf16 ? launch_flush_ragged_fmt<false, true>(a, stream) : launch_flush_ragged_fmt<false, false>(a, stream);
}

template <int BITS, bool KEYS, bool BF16>
static hipError_t launch_dequant_ragged_t(const DequantArgs& a, hipStream_t stream) {
    const int64_t per_bh = (a.n + kG - 1) / kG;
    const int64_t n_tiles = a.BH * per_bh;
    const int64_t blocks = (n_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL((dequant_ragged_kernel<BITS, KEYS, BF16>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kBlock), 0, stream, a.codes, a.codes_bh_stride,
                       static_cast<const float*>(a.scale), static_cast<const float*>(a.zero),
                       a.meta_bh_stride, a.t0, a.n, a.out, a.out_bh_stride, per_bh, n_tiles, a.head_dim);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_dequant_ragged_fmt(const DequantArgs& a, hipStream_t stream) {
    const bool keys = a.kind == KIVI_KEYS;
    if (a.bits == 4) return keys ? launch_dequant_ragged_t<4, true, BF16>(a, stream)
                                 : launch_dequant_ragged_t<4, false, BF16>(a, stream);
    return keys ? launch_dequant_ragged_t<2, true, BF16>(a, stream)
                : launch_dequant_ragged_t<2, false, BF16>(a, stream);
}

hipError_t launch_dequant_ragged(const DequantArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_dequant_ragged_fmt<true>(a, stream) : launch_dequant_ragged_fmt<false>(a, stream);
}

}  // namespace kivi
