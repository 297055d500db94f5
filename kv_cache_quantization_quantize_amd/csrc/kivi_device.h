// kivi_device.h -- device-side helpers shared by the libkivi kernels
// (internal to the library; not part of the C ABI).
//
// Geometry of the flush and dequantize (wave64): a "tile" is 32 consecutive
// tokens (a key flush tile: one whole group of G tokens) x D channels of one
// bh slab.  A token row is D/8 lanes of 8 channels (RowGeo below), so lane l
// holds channels 8*(l % (D/8)) .. +7 of tokens tile_start + l/(D/8) + i*64/(D/8):
// each token row is read as one contiguous segment of 2*D bytes and every
// load instruction of the wave covers 1 KiB of consecutive rows.  At the
// default head_dim 128 that is 16 lanes per row and 4 rows per load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace kivi {

constexpr int kHeadDim = 128;      // the decode-loop cache's head_dim (rows it copies)
constexpr int kGroup = 32;         // the cache's group size; the attend's smallest
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;

// Exact widening of the low / high bfloat16 of a 32-bit word (bfloat16 is
// binary32 with the low 16 fraction bits dropped).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> fp16, round to nearest even (the default rounding mode).
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Streaming accesses: the flush and dequantize read their inputs and write
// their outputs exactly once, so they carry the nontemporal hint (it kept
// the full-cache key and value flushes 5-8% faster in a side-by-side run).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store_stream(uint16_t* p, const uint4& v) {
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream4(float* p, float a, float b, float c, float d) {
    __builtin_nontemporal_store(f32x4_t{a, b, c, d}, reinterpret_cast<f32x4_t*>(p));
}

__device__ __forceinline__ uint4 pack8(const uint32_t (&h)[8]) {
    uint4 v;
    v.x = h[0] | (h[1] << 16);
    v.y = h[2] | (h[3] << 16);
    v.z = h[4] | (h[5] << 16);
    v.w = h[6] | (h[7] << 16);
    return v;
}

// Two fp16 values in one VGPR, for the packed min/max instructions.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// IEEE 754-2019 minimum/maximum: exact on finite values, -0 < +0 (zeros are
// canonicalized afterwards).  Three inputs map to v_pk_minimum3_f16 /
// v_pk_maximum3_f16.
__device__ __forceinline__ half2_t hmin(half2_t a, half2_t b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ half2_t hmax(half2_t a, half2_t b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ half2_t hmin3(half2_t a, half2_t b, half2_t c) { return hmin(hmin(a, b), c); }
__device__ __forceinline__ half2_t hmax3(half2_t a, half2_t b, half2_t c) { return hmax(hmax(a, b), c); }

// Reductions across the four 16-lane rows of a wave with the gfx950 lane
// swaps: permlane16_swap exchanges rows 0<->1 and 2<->3, permlane32_swap the
// two halves, so min(a, b) of the two swapped copies combines row pairs.
__device__ __forceinline__ half2_t row_pair_min(half2_t v) {
    const auto p = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
    return hmin(as_h2(p[0]), as_h2(p[1]));
}
__device__ __forceinline__ half2_t row_pair_max(half2_t v) {
    const auto p = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
    return hmax(as_h2(p[0]), as_h2(p[1]));
}
__device__ __forceinline__ half2_t half_min(half2_t v) {
    const auto p = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return hmin(as_h2(p[0]), as_h2(p[1]));
}
__device__ __forceinline__ half2_t half_max(half2_t v) {
    const auto p = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return hmax(as_h2(p[0]), as_h2(p[1]));
}

// fp32 forms of the same: IEEE minimum/maximum (v_minimum3_f32 /
// v_maximum3_f32 for three inputs).
__device__ __forceinline__ float fminimum(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float fmaximum(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmin3(float a, float b, float c) { return fminimum(fminimum(a, b), c); }
__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaximum(fmaximum(a, b), c); }
// Word k (0..3) of a 16-byte load: channels 2k and 2k+1 of the lane's 8.
__device__ __forceinline__ uint32_t word_of(const uint4& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Row geometry of the flush and dequantize for head_dim D: a token row is
// D/8 chunks of 8 channels, one per lane, in a row of 8, 16 or 32 lanes (the
// next power of two; head_dims 96, 160, 192 and 224 leave the last lanes of
// a row idle), so one wave covers 8, 4 or 2 rows per load.  The lanes that
// hold the same 8 channels of different rows are lane ^ 8 (rows of 8 only),
// ^ 16 (rows of 8 or 16) and ^ 32.
template <int D>
struct RowGeo {
    static constexpr int kChunks = D / 8;          // lanes of a row that hold channels
    static constexpr int kLanesPerRow = kChunks <= 8 ? 8 : kChunks <= 16 ? 16 : 32;
    static constexpr int kRowsPerWave = 64 / kLanesPerRow;
};

// lane ^ 8 within each row of 16: DPP row_ror:8
__device__ __forceinline__ uint32_t lane_xor8(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, false));
}

// min / max over the rows of a wave for each lane's channel block
template <int D>
__device__ __forceinline__ half2_t cross_rows_min(half2_t v) {
    if constexpr (RowGeo<D>::kLanesPerRow == 8) v = hmin(v, as_h2(lane_xor8(as_u32(v))));
    if constexpr (RowGeo<D>::kLanesPerRow <= 16) v = row_pair_min(v);
    return half_min(v);
}
template <int D>
__device__ __forceinline__ half2_t cross_rows_max(half2_t v) {
    if constexpr (RowGeo<D>::kLanesPerRow == 8) v = hmax(v, as_h2(lane_xor8(as_u32(v))));
    if constexpr (RowGeo<D>::kLanesPerRow <= 16) v = row_pair_max(v);
    return half_max(v);
}
template <int D>
__device__ __forceinline__ float cross_rows_min_f32(float v) {
    if constexpr (RowGeo<D>::kLanesPerRow == 8) v = fminimum(v, __uint_as_float(lane_xor8(__float_as_uint(v))));
    if constexpr (RowGeo<D>::kLanesPerRow <= 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fminimum(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fminimum(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
template <int D>
__device__ __forceinline__ float cross_rows_max_f32(float v) {
    if constexpr (RowGeo<D>::kLanesPerRow == 8) v = fmaximum(v, __uint_as_float(lane_xor8(__float_as_uint(v))));
    if constexpr (RowGeo<D>::kLanesPerRow <= 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// DPP quad permutations (lane ^ 1, lane ^ 2 within each group of 4 lanes).
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false));
}
// DPP mirrors within each half-row of 8 lanes (lane i <- 7 - i) and within
// each row of 16 (lane i <- 15 - i): after the quad exchanges every lane of a
// quad holds the quad's value, so one mirror joins two quads (8 lanes) and a
// second joins two half-rows (16 lanes).
__device__ __forceinline__ uint32_t half_row_mirror(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t row_mirror(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x140, 0xF, 0xF, false));
}

// scale = RN(range / (2^bits - 1)) in three operations: a product with the
// rounded reciprocal of the constant, then one FMA correction step.  This
// equals the IEEE quotient for every binary32 range in [2^-24, 2^18) and for
// 0, checked exhaustively for both divisors (every range here is 0 or a
// rounded difference of two fp16 values, so it lies in that set).
template <int BITS>
__device__ __forceinline__ float scale_of(float range) {
    constexpr float kL = static_cast<float>((1 << BITS) - 1);
    constexpr float kRL = 1.0f / kL;
    const float q0 = range * kRL;
    const float rho = __builtin_fmaf(-q0, kL, range);
    return __builtin_fmaf(rho, kRL, q0);
}

// 1/s to within 2^-22 relative: hardware reciprocal r0 plus one Newton step
// e = RN(1 - s*r0), r1 = RN(r0 + r0*e).  The step squares r0's relative
// error (any r0 within 2^-12 leaves at most 2^-24) and its two roundings add
// at most 2^-23.  A constant group (s = 0) gets r = 2^126 from the clamp, and
// all its t are 0, so its products are exactly 0 (no 0 * inf).  Every
// non-zero scale is >= 2^-24/15 > 2^-126, so the clamp changes nothing else.
__device__ __forceinline__ float recip_clamped(float s) {
    const float sc = fmaxf(s, 0x1p-126f);
    const float r0 = __builtin_amdgcn_rcpf(sc);
    const float e = __builtin_fmaf(-sc, r0, 1.0f);
    return __builtin_fmaf(r0, e, r0);
}

// t = x - zero from the fp16 input in one mixed-precision FMA.  `one` is a
// kernel argument equal to 1.0f: x*1 is exact, so this is the IEEE
// subtraction of the widened input (the compiler would fold a literal 1.0
// into a separate conversion and subtraction).
__device__ __forceinline__ float sub_from_f16(_Float16 x, float one, float zero) {
    return __builtin_fmaf(static_cast<float>(x), one, -zero);
}

// Code of one element on the fast path: q = rint(t * r), and |y - q| is folded
// into `dev` (the largest distance of the row's quotients from their integer).
//
// Why q equals rint(fl(t / s)) when every |y - q| <= 1/2 - 2^-16.  With
// |r - 1/s| <= 2^-22/s, y = RN(t*r) and z = t/s < 16:
//   |y - z| <= z (2^-22 + 2^-24) (1 + 2^-22),  |fl(z) - z| <= z 2^-24,
// so |y - fl(z)| < 16 * 1.51 * 2^-22 < 2^-17.  rint only changes value at
// half-integers, so if y is farther than 2^-16 from every half-integer,
// y and fl(z) round to the same integer; otherwise the caller recomputes the
// row with the IEEE quotient.  (y - q is exact: q = rint(y) is within half
// of y.)  The code needs no clip: 0 <= t <= range (rounding is monotone) and
// s >= (range/L)(1 - 2^-24) bound y by L (1 + 2^-21) < L + 1/2.
__device__ __forceinline__ float quant_fast(float t, float r, float& dev) {
    const float y = t * r;
    const float q = __builtin_rintf(y);
    dev = fmaxf(dev, __builtin_fabsf(y - q));
    return q;
}
constexpr float kNearTie = 0.5f - 0x1p-16f;

// The same code with the IEEE quotient (the oracle's exact steps); t = x - zero.
// The clip to [0, 2^bits - 1] is a no-op (see quant_fast: 0 <= t <= range
// and s is the rounded range/L); it is kept so these are the oracle's steps
// for every input, fp16 or bfloat16.
__device__ __forceinline__ float quant_exact(float t, float s, float levels) {
    if (s == 0.0f) return 0.0f;
    return fminf(fmaxf(__builtin_rintf(t / s), 0.0f), levels);
}

// t = x - zero for element j (0..7) of a lane's 16-byte row: fp16 through
// sub_from_f16, bfloat16 widened exactly and subtracted in fp32.
template <bool BF16>
__device__ __forceinline__ float sub_elem(const uint4& raw, int j, float one, float zero) {
    const uint32_t w = word_of(raw, j >> 1);
    if constexpr (BF16) {
        return ((j & 1) ? bf16_hi(w) : bf16_lo(w)) - zero;
    } else {
        return sub_from_f16(as_h2(w)[j & 1], one, zero);
    }
}

// A zero extreme is stored as +0, so the result does not depend on which
// signed zero a reduction kept: -0 + 0 = +0 in round-to-nearest, and v + 0 = v
// for every other v.
__device__ __forceinline__ float canon_zero(float v) { return v + 0.0f; }

// Reconstruction fp16_rne(fl(fl(q * scale) + zero)) -- two roundings, no FMA.
__device__ __forceinline__ uint32_t recon_f16(float q, float scale, float zero) {
    const float prod = q * scale;
    const float sum = prod + zero;
    return f32_to_f16(sum);
}

// ---------------------------------------------------------------------------
// bfloat16 storage: binary32 with the low 16 fraction bits dropped.
// ---------------------------------------------------------------------------

// fp32 -> bfloat16, round to nearest even on the bit pattern: adding
// 0x7fff plus the lowest kept bit rounds the dropped half up past the
// midpoint, and at the midpoint only when that would make the kept part
// even; a carry moves into the exponent (up to infinity), which is the
// correct rounding too.  Exact for every finite input, subnormals included.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Reconstruction bf16_rne(fl(fl(q * scale) + zero)).
__device__ __forceinline__ uint32_t recon_bf16(float q, float scale, float zero) {
    const float prod = q * scale;
    const float sum = prod + zero;
    return f32_to_bf16(sum);
}

template <bool BF16>
__device__ __forceinline__ uint32_t recon_out(float q, float scale, float zero) {
    if constexpr (BF16) return recon_bf16(q, scale, zero);
    else return recon_f16(q, scale, zero);
}

// The scale for bfloat16 inputs.  scale_of is proven equal to the IEEE
// quotient for every binary32 range in {0} and [2^-24, 2^18); bfloat16
// ranges can lie anywhere in the binary32 exponent range, so a wave takes
// the plain IEEE quotient whenever one of its lanes has a range outside
// that set (the branch is uniform, and not taken for ordinary caches).
template <int BITS>
__device__ __forceinline__ float scale_wide(float range) {
    const bool proven = range == 0.0f || (range >= 0x1p-24f && range < 0x1p18f);
    if (__builtin_amdgcn_ballot_w64(!proven) == 0) return scale_of<BITS>(range);
    return range / static_cast<float>((1 << BITS) - 1);
}

// The reciprocal fast path of quant_fast needs a normal scale with a normal
// reciprocal; any other scale (zero included) takes the IEEE quotient.
__device__ __forceinline__ bool fast_scale(float s) { return s >= 0x1p-126f && s < 0x1p126f; }

// ---------------------------------------------------------------------------
// Binary16 scale/zero: the binary32 scale rounded to nearest even binary16
// is what the store holds and what the codes and reconstruction use.  (The
// zero of an fp16 group is an fp16 value and needs no rounding.)
// ---------------------------------------------------------------------------
//
// The empty asm keeps s a rounded binary32 value.  Without it the compiler
// folds the FMA that produces s (the last step of scale_of) and this
// conversion into one mixed-precision FMA with a binary16 result, which
// rounds once instead of twice: RN16(x) differs from RN16(RN32(x)) wherever
// RN32(x) lands exactly on a binary16 midpoint, and the store would then
// hold a different scale than the reading defines.
__device__ __forceinline__ float round_to_f16(float s) {
    __asm__("" : "+v"(s));
    return static_cast<float>(static_cast<_Float16>(s));
}

// quant_fast's bounds hold for a normal binary16 scale: it is within 2^-11
// (relative) of the binary32 one, so t / s <= L (1 + 2^-10) stays below
// L + 1/2 and below 16, and no clip is needed.  A non-constant group whose
// scale rounded to a subnormal or to 0 takes quant_exact (IEEE quotient and
// clip; code 0 for a zero scale).  A constant group keeps the fast path: its
// t are all 0.
__device__ __forceinline__ bool slow_scale16(float s, float range) { return range != 0.0f && s < 0x1p-14f; }

}  // namespace kivi
