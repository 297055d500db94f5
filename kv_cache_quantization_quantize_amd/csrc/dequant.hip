// dequant.hip -- expand a packed key or value store back to fp16 (or
// bfloat16) for a token range: out = rne(fl(fl(q * scale) + zero)), the same
// two roundings as
// the flush's reconstruction (blog post "A 5.65x Metal Kernel That Made My
// LLM Exactly 0% Faster", "Three ways to be off by one bit", item 1; "So why
// does the kernel ship?": the shipped cache expands to fp16 before
// attention).
//
// One wave per 32-token x 128-channel tile with the lane mapping of
// kivi_device.h: per token a lane reads one code word (4-bit) or half a word
// (2-bit) and writes 16 contiguous bytes of fp16.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

// Workgroups per CU a dequantize launch is held to by LDS it reserves and
// never touches (160 KiB per CU on gfx950; 0: no cap).  Measured on the
// full 32k cache, interleaved against full residency: 5 per CU ran the fp16
// dequantizes 1-3% faster at 4 bits and 5-11% faster at 2 bits and at
// head_dim 96; bfloat16 values gained 1-2% at 4 per CU and bfloat16 keys
// lost 1-2% with any cap.  Before every row's loads were issued ahead of the
// first store, a cap of 3 or 4 per CU had doubled the value dequantize's
// time (one memory round trip per row, hidden only by many waves).
template <bool KEYS, bool BF16> constexpr int kDequantPerCU = BF16 ? (KEYS ? 0 : 4) : 5;

// Eight consecutive scale (or zero) entries as floats: binary32, or binary16
// widened exactly.  p is 16-byte aligned (the ABI's slab stride and head_dim
// rows keep it so).
__device__ __forceinline__ void load_meta8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load_meta8(const uint16_t* p, float (&v)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const half2_t h = as_h2(word_of(a, k));
        v[2 * k] = static_cast<float>(h[0]);
        v[2 * k + 1] = static_cast<float>(h[1]);
    }
}
__device__ __forceinline__ float meta_value(float m) { return m; }
__device__ __forceinline__ float meta_value(uint16_t m) { return static_cast<float>(__builtin_bit_cast(_Float16, m)); }

// Rows [0, n_rows) of one tile; row k is store token t_first + k, written to
// ot + k*128.  ONE_GROUP (keys only): the 32 rows are exactly one key group,
// so its scale and zero are loaded once for the tile.
template <int BITS, bool KEYS, bool ONE_GROUP, bool BF16, int G, int D, typename MT>
__device__ __forceinline__ void dequant_tile(const uint32_t* __restrict__ cb, const MT* __restrict__ scb,
                                             const MT* __restrict__ zeb, int64_t t_first, int n_rows,
                                             uint16_t* __restrict__ ot, int lane)
{
    constexpr int kWords = D * BITS / 32;
    constexpr uint32_t kMask = (1u << BITS) - 1u;
    constexpr int kMetaPerTok = (D + G - 1) / G;   // value groups per token (the last may be short)
    constexpr int kLPR = RowGeo<D>::kLanesPerRow;
    constexpr int kRPW = RowGeo<D>::kRowsPerWave;
    constexpr int kChunks = RowGeo<D>::kChunks;
    const int c = lane % kLPR;
    const int r = lane / kLPR;
    // lanes past a row's last chunk (head_dims that are not 64, 128 or 256)
    // have nothing to write, and no lane exchanges follow
    if (kChunks != kLPR && c >= kChunks) return;
    const uint32_t* ct = cb + t_first * kWords;
    float gs[8], gz[8];
    if constexpr (ONE_GROUP) {
        load_meta8(scb + (t_first / G) * D + c * 8, gs);
        load_meta8(zeb + (t_first / G) * D + c * 8, gz);
    }
    constexpr int kIters = 32 / kRPW;
    // Every row's code word (and, for values, its group's scale and zero) is
    // loaded before the first store, rows past n_rows re-reading the last
    // one, so a tile costs one memory round trip rather than one per row.
    uint32_t wv[kIters];
    float vs[kIters], vz[kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int k = min(r + kRPW * i, n_rows - 1);
        if constexpr (BITS == 4) wv[i] = ct[k * kWords + c];
        else wv[i] = ct[k * kWords + (c >> 1)] >> (16 * (c & 1));
        if constexpr (!KEYS) {
            const int64_t t = t_first + k;
            vs[i] = meta_value(scb[t * kMetaPerTok + c / (G / 8)]);
            vz[i] = meta_value(zeb[t * kMetaPerTok + c / (G / 8)]);
        }
    }
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int k = r + kRPW * i;                    // output row
        if (!ONE_GROUP && k >= n_rows) continue;
        const uint32_t w = wv[i];
        float sc[8], ze[8];
        if constexpr (ONE_GROUP) {
#pragma unroll
            for (int j = 0; j < 8; ++j) { sc[j] = gs[j]; ze[j] = gz[j]; }
        } else if constexpr (KEYS) {
            // a tile that straddles key groups (an unaligned window)
            const int64_t t = t_first + k;
            load_meta8(scb + (t / G) * D + c * 8, sc);
            load_meta8(zeb + (t / G) * D + c * 8, ze);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) { sc[j] = vs[i]; ze[j] = vz[i]; }
        }
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = recon_out<BF16>(static_cast<float>((w >> (BITS * j)) & kMask), sc[j], ze[j]);
        store_stream(ot + k * D + c * 8, pack8(h));
    }
}

template <int BITS, bool KEYS, bool BF16, int G, int D, typename MT>
__global__ __launch_bounds__(kBlock) void dequant_kernel(
    const uint32_t* __restrict__ codes, int64_t codes_bh_stride,
    const MT* __restrict__ scale, const MT* __restrict__ zero, int64_t meta_bh_stride,
    int64_t t0, int64_t n, uint16_t* __restrict__ out, int64_t out_bh_stride,
    int64_t tiles_per_bh, int64_t n_tiles)
{
    const int lane = threadIdx.x & 63;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;                   // uniform across the wave

    const int64_t bh = tile / tiles_per_bh;
    const int64_t i0 = (tile - bh * tiles_per_bh) * 32;
    const int64_t rows = n - i0;
    const uint32_t* cb = codes + bh * codes_bh_stride;
    const MT* scb = scale + bh * meta_bh_stride;
    const MT* zeb = zero + bh * meta_bh_stride;
    uint16_t* ot = out + bh * out_bh_stride + i0 * D;
    // a full tile inside one key group loads the group's scale and zero once
    if (KEYS && rows >= 32 && (t0 + i0) % G + 32 <= G)
        dequant_tile<BITS, KEYS, true, BF16, G, D, MT>(cb, scb, zeb, t0 + i0, 32, ot, lane);
    else
        dequant_tile<BITS, KEYS, false, BF16, G, D, MT>(cb, scb, zeb, t0 + i0, rows < 32 ? static_cast<int>(rows) : 32, ot, lane);
}

template <int BITS, bool KEYS, bool BF16, int G, int D, typename MT>
static hipError_t launch_t(const DequantArgs& a, hipStream_t stream) {
    const int64_t tiles_per_bh = (a.n + 31) / 32;
    const int64_t n_tiles = a.BH * tiles_per_bh;
    const int64_t blocks = (n_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    constexpr int kPerCU = kDequantPerCU<KEYS, BF16>;
    const size_t lds = kPerCU > 0 ? (size_t{160} * 1024 / kPerCU) / 1024 * 1024 : 0;
    hipLaunchKernelGGL((dequant_kernel<BITS, KEYS, BF16, G, D, MT>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kBlock), lds, stream, a.codes, a.codes_bh_stride,
                       static_cast<const MT*>(a.scale), static_cast<const MT*>(a.zero),
                       a.meta_bh_stride, a.t0, a.n, a.out, a.out_bh_stride, tiles_per_bh, n_tiles);
    return hipGetLastError();
}

template <bool BF16, int G, int D, typename MT = float>
static hipError_t launch_g(const DequantArgs& a, hipStream_t stream) {
    const bool keys = a.kind == 0;
    if (a.bits == 4) return keys ? launch_t<4, true, BF16, G, D, MT>(a, stream) : launch_t<4, false, BF16, G, D, MT>(a, stream);
    return keys ? launch_t<2, true, BF16, G, D, MT>(a, stream) : launch_t<2, false, BF16, G, D, MT>(a, stream);
}

// head_dim 128 with groups of 32, 64 or 128; every other multiple of 16 up
// to 256 with groups of 32.  Binary16 metadata: fp16 output at head_dim 128.
template <bool BF16>
static hipError_t launch_fmt(const DequantArgs& a, hipStream_t stream) {
    switch (a.head_dim) {
#define KIVI_DEQUANT_D(D) case D: return launch_g<BF16, 32, D>(a, stream);
        KIVI_DEQUANT_D(16) KIVI_DEQUANT_D(32) KIVI_DEQUANT_D(48) KIVI_DEQUANT_D(64) KIVI_DEQUANT_D(80)
        KIVI_DEQUANT_D(96) KIVI_DEQUANT_D(112) KIVI_DEQUANT_D(144) KIVI_DEQUANT_D(160) KIVI_DEQUANT_D(176)
        KIVI_DEQUANT_D(192) KIVI_DEQUANT_D(208) KIVI_DEQUANT_D(224) KIVI_DEQUANT_D(240) KIVI_DEQUANT_D(256)
#undef KIVI_DEQUANT_D
        default: break;
    }
    if constexpr (!BF16) {
        if (a.meta16) {
            switch (a.group) {
                case 64: return launch_g<false, 64, 128, uint16_t>(a, stream);
                case 128: return launch_g<false, 128, 128, uint16_t>(a, stream);
                default: return launch_g<false, 32, 128, uint16_t>(a, stream);
            }
        }
    }
    switch (a.group) {
        case 64: return launch_g<BF16, 64, 128>(a, stream);
        case 128: return launch_g<BF16, 128, 128>(a, stream);
        default: return launch_g<BF16, 32, 128>(a, stream);
    }
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream) {
    // every head_dim the ABI admits (multiples of 16 up to 256) on the tiled
    // kernel, as the flush; the ABI rejects the others before any launch
    if (a.head_dim < 16 || a.head_dim > 256 || a.head_dim % 16 != 0) return hipErrorInvalidValue;
    return a.bf16 ? launch_fmt<true>(a, stream) : launch_fmt<false>(a, stream);
}

}  // namespace kivi
