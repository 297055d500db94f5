// attend_device.h -- device code of the fused dequantize + attend for one
// new query token per sequence over a packed 2/4-bit store plus a 16-bit
// residual window (internal; included by attend.hip for fp16 caches and by
// attend_bf16.hip for bfloat16 caches, so the two compile in parallel).
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
// Design for MI355X: one wave per (sequence, kv head, token split).  The
// wave serves every query head that shares the kv head, so each packed
// byte is read from HBM once; the token axis is split so the grid reaches
// thousands of workgroups even at B=1 (which answers the occupancy limit the
// pages measured).  Partials (m, l, o[128]) go to the workspace and a second
// kernel merges them with the log-sum-exp rule.
//
// Arithmetic: QK^T and PV run on MFMA (fp32 accumulation) with operands in
// the cache's 16-bit format, fp16 or bfloat16 (template parameter BF).  K and
// V are dequantized in registers to that format with one FMA per element
// (within one rounding of the stored reconstruction); q enters exactly,
// softmax probabilities are rounded to the same format for PV, and the
// online softmax runs in fp32, base 2.
//
// Grid: one 64-lane wave per (sequence, kv head, split of the token axis);
// each wave walks its split in 32-token steps, one key group per step, with
// the step's key and value metadata staged through LDS.
#pragma once

#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// 8 fp16 or bfloat16 values in 4 VGPRs: one MFMA operand of one lane.
union Frag {
    half8_t h;
    bf16x8_t b;
    uint32_t u[4];
};

// D += A B for one 16x16x32 tile, fp16 or bfloat16 operands (same lane
// layout, below).
template <bool BF>
__device__ __forceinline__ float4_t mfma(const Frag& a, const Frag& b, float4_t c) {
    if constexpr (BF) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.b, b.b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.h, b.h, c, 0, 0, 0);
}

#ifndef KIVI_ATTEND_NBUF
#define KIVI_ATTEND_NBUF 2
#endif
#define KIVI_ATTEND_OCCUPANCY __attribute__((amdgpu_waves_per_eu(KIVI_ATTEND_WAVES_PER_SIMD)))
constexpr int kNBuf = KIVI_ATTEND_NBUF;

constexpr int kStep = kAttendStep;    // tokens per wave step (one key group)
constexpr float kLog2e = 1.4426950408889634f;
// The code-to-float trick: a code masked into the low mantissa bits under the
// exponent of M reads as M + code exactly.  fp16 (10 fraction bits): M =
// 1024; bfloat16 (7 fraction bits): M = 128.
template <bool BF> constexpr uint32_t kMagic = BF ? 0x43004300u : 0x64006400u;   // M in both halves
template <bool BF> constexpr float kMagicValue = BF ? 128.0f : 1024.0f;

// v_mfma_f32_16x16x32_f16 lane layout (gfx950, wave64), lane l = 16*q + n:
//   A (16x32): lane l holds row m = n, columns 8q .. 8q+7 (slot s = column - 8q)
//   B (32x16): lane l holds rows 8q .. 8q+7, column n
//   D (16x16 fp32): lane l holds rows 4q .. 4q+3, column n
// The product only pairs A slot s of lane (q, m) with B slot s of lane (q, n),
// so any bijection channel <-> (q, slot) used on both sides is valid.
//
// Channel order inside an 8-channel unit: the codes of channels j and j+4
// come out of one SIMD-within-register extraction, so slot 2j holds channel
// j and slot 2j+1 channel j+4 (j = 0..3).  Key unit kb of lane group q is
// channels 32q + 8kb .. 32q + 8kb + 7.

// (x & mask) | magic in one v_bitop3_b32 (truth table 0xEA = (a & b) | c).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
    return __builtin_amdgcn_bitop3_b32(x, mask, magic, 0xEA);
}

// Four 16-bit pairs from the 8 codes of one 8-channel unit: pair j holds the
// codes of channels j and j+4.  A code masked in place at bit offset e of
// the mantissa under the exponent of M reads as M + 2^e code exactly, so no
// shift is needed while the code stays inside the fraction bits; the factor
// 2^-e goes into the staged scale (kscale_factor).  fp16, 4-bit: one code
// word, e = 4 (j & 1) after one shift by 8 for j >= 2; bfloat16 keeps every
// nibble at e = 0 (bits 4..7 would reach its exponent), with shifts by 4, 8
// and 12.  2-bit: the unit's half of a word spread to bytes 0 and 2 first,
// e = 2 j (fp16) or min(2 j, 4) (bfloat16, one more shift for j = 3).
template <int BITS, bool BF>
__device__ __forceinline__ void code_pairs(uint32_t w, int half, uint32_t (&p)[4]) {
    constexpr uint32_t kM = kMagic<BF>;
    if constexpr (BITS == 4) {
        if constexpr (BF) {
            p[0] = and_or(w, 0x000F000Fu, kM);
            p[1] = and_or(w >> 4, 0x000F000Fu, kM);
            p[2] = and_or(w >> 8, 0x000F000Fu, kM);
            p[3] = and_or(w >> 12, 0x000F000Fu, kM);
        } else {
            const uint32_t w8 = w >> 8;
            p[0] = and_or(w, 0x000F000Fu, kM);
            p[1] = and_or(w, 0x00F000F0u, kM);
            p[2] = and_or(w8, 0x000F000Fu, kM);
            p[3] = and_or(w8, 0x00F000F0u, kM);
        }
    } else {
        const uint32_t sel = half ? 0x0C030C02u : 0x0C010C00u;
        const uint32_t x = __builtin_amdgcn_perm(w, w, sel);
#pragma unroll
        for (int j = 0; j < 3; ++j) p[j] = and_or(x, 0x00030003u << (2 * j), kM);
        p[3] = BF ? and_or(x >> 2, 0x00300030u, kM) : and_or(x, 0x00C000C0u, kM);
    }
}

// 2^-e for key channel c (c & 3 = j is its pair in the unit, see code_pairs).
template <int BITS, bool BF>
__device__ __forceinline__ float kscale_factor(int c) {
    if constexpr (BITS == 4) return (!BF && (c & 1)) ? 0.0625f : 1.0f;
    else return __builtin_ldexpf(1.0f, -(BF ? min(2 * (c & 3), 4) : 2 * (c & 3)));
}

// bfloat16 caches at 4 bits take another route to the key and value
// operands: the two nibbles of every byte of a code word are split into
// byte lanes (one AND, and one shift and AND, per word), each byte becomes
// an fp32 integer c in one v_cvt_f32_ubyte*, and the element is
// RN32(c s + z) rounded to bfloat16 (no magic offset, so zero is used as
// stored).  Channels then pair as (2j, 2j+1), so the query and the
// residual key operands keep their natural channel order on this route.
template <int BITS, bool BF> constexpr bool kByteCodes = BF && BITS == 4;
// The offset the staged zero absorbs: M for the magic-number routes, 0 for
// the byte route.
template <int BITS, bool BF> constexpr float kCodeOffset = kByteCodes<BITS, BF> ? 0.0f : kMagicValue<BF>;

// Byte k of x as an exact fp32 integer (one v_cvt_f32_ubyte{k}).
__device__ __forceinline__ float byte_f32(uint32_t x, int k) {
    return static_cast<float>(static_cast<uint8_t>(x >> (8 * k)));
}

// The nibbles of a code word split into byte lanes: even nibbles (lo) and
// odd ones (hi).  The empty asm hides the masks from the optimizer, which
// would otherwise fold each later byte extraction into a bit-field extract
// plus a conversion instead of one v_cvt_f32_ubyte{k}.
__device__ __forceinline__ void split_nibbles(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = w & 0x0F0F0F0Fu;
    hi = (w >> 4) & 0x0F0F0F0Fu;
    __asm__("" : "+v"(lo), "+v"(hi));
}

// Two fp32 values rounded to one bfloat16 pair (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    bf16x2_t r;
    r[0] = static_cast<__bf16>(a);
    r[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, r);
}

// code * scale + zero as one mixed-precision FMA with an fp16 result:
// c16 = 1024 + code exactly and zp = RN32(zero - 1024 s), so the result is
// code*s + zero up to 2^-24 (|zero| + 1024 s) plus the fp16 rounding (the
// attend is checked against the float64 definition to 2e-3, not bit-exactly).
// Both halves of one fp16 pair register: lo = fma(c.lo, s0, z0), hi =
// fma(c.hi, s1, z1), each rounded to fp16.  Written in C, not inline asm, so
// the compiler sees the register writes and keeps the wait states an MFMA
// needs after a VALU write of its operands.
// bfloat16 (BF): c = 128 + code widened by a shift, one fp32 FMA each, and
// the pair rounded to bfloat16 (nearest even).
template <bool BF>
__device__ __forceinline__ uint32_t deq2(uint32_t pair, float s0, float z0, float s1, float z1) {
    if constexpr (BF) {
        return bf16_pair(__builtin_fmaf(__uint_as_float(pair << 16), s0, z0),
                         __builtin_fmaf(__uint_as_float(pair & 0xffff0000u), s1, z1));
    } else {
        const half2_t c = as_h2(pair);
        half2_t r;
        r[0] = static_cast<_Float16>(__builtin_fmaf(static_cast<float>(c[0]), s0, z0));
        r[1] = static_cast<_Float16>(__builtin_fmaf(static_cast<float>(c[1]), s1, z1));
        return as_u32(r);
    }
}

// lane exchanges across the four 16-lane rows (see kivi_device.h)
__device__ __forceinline__ float rows_max(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __builtin_elementwise_maximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
    p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// The slab of one (sequence, kv head) as raw buffer resources whose extent
// ends at store token n_quant: a load past the extent returns zero, so the
// masked tokens of a partial last step read finite zeros and no load leaves
// the slab.  Word 3 is the raw-buffer format of gfx9-family parts (32-bit
// data format, no swizzle, no thread-id indexing).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy operand of the store loads: the nontemporal hint (`nt` on
// gfx950).  A call reads each packed byte once; with the hint the B=32,
// 16384-token attend ran 7-8% faster in a side-by-side run.
constexpr int kStreamLoad = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// A step start whose every load lies past the buffers' extent: the ABI
// keeps n_quant below 2^24 tokens, and every buffer's offset for token t is
// t times its bytes per token (key metadata: per token of the group), so a
// start at 1.5 x 2^24 lands at 1.5 times any buffer's largest extent.  The
// largest such offset is 1.5 x 2^24 x 128 B (the code rows of head_dim 256
// at 4 bits) = 3 x 2^30, so lane and instruction offsets (under 2^13) keep
// every one of them below 2^32 (a start of 2^25 wrapped to the slab's first
// rows there).
constexpr uint32_t kFarToken = 3u << 23;
static_assert(kFarToken > (1u << 24), "a far step must start past every extent (n_quant < 2^24)");
static_assert(uint64_t{kFarToken} * 128 + (1u << 13) < (uint64_t{1} << 32),
              "far offsets of 128-byte code rows plus lane offsets must not wrap");

struct StoreView {
    rsrc_t kc, ks, kz;      // key codes, scale, zero
    rsrc_t vc, vs, vz;      // value codes, scale, zero
};

// Byte offsets of a lane's loads at step t0 = 0; a step adds t0 times the
// bytes per token (key metadata: t0 / G groups of 128 pairs).
struct LaneOffsets {
    uint32_t k;             // key codes of token n, the lane's 32 channels
    uint32_t v;             // value code word of token 4q, the lane's 8 channels
    uint32_t km;            // key scale / zero of channels 2l, 2l+1
    uint32_t vm;            // value scale / zero of token l & 31: groups 2(l>>5), +1 (G = 32),
                            // groups 0, 1 (G = 64) or group 0 (G = 128)
    // Padded kernels: whether the lane's key code, value code and key
    // metadata channels reach below the store's head_dim.  The loads of a
    // lane that holds only padded channels go to kDeadOffset instead.
    bool k_live = true, v_live = true, km_live = true;
};

// A buffer offset past every extent (the ABI keeps extents below 2^31): a
// load there returns zeros without a memory access.  Instruction offsets of
// at most 16 keep it below 2^32.
constexpr uint32_t kDeadOffset = 0xFFFFFF00u;
static_assert(uint64_t{kDeadOffset} + 32 < (uint64_t{1} << 32) && kDeadOffset > (1u << 31),
              "dead loads must stay past every extent without wrapping");

// Channel geometry for head_dim D (64, 128 or 256).  QK^T: lane group q
// holds channels kCPG*q + 8*kb + slot of key unit kb < kKB.  PV: MFMA i < kPV
// covers channels kPV*m + i (m = 0..15), so lane (q, n) takes the kPV
// channels kPV*n .. kPV*n + kPV - 1 of its tokens.  Lane l stages the key
// scale/zero of kKMC channels (kKMC*l .. kKMC*l + kKMC - 1, lanes past D/kKMC
// idle) and the value scale/zero of token l & 31, kVMG of its groups.
template <int D> struct Geo {
    static constexpr int kCPG = D / 4;          // channels per 16-lane group
    static constexpr int kKB = D / 32;          // QK^T key units (MFMA k-steps)
    static constexpr int kPV = D / 16;          // PV MFMAs
    static constexpr int kKMC = D == 256 ? 4 : 2;
};

// The words of a lane's scale (or zero) load for staging: four channels or
// groups at head_dim 256 (binary32 only), two otherwise.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int N> struct MetaWords { typedef u32x2 type; };
template <> struct MetaWords<4> { typedef u32x4 type; };

// Loads of one 32-token step of store tokens, issued one step ahead of the
// compute that uses them.
// Scale and zero stay as loaded (binary32 pairs, or binary16 pairs in the
// low word) until the step that uses them, so that issuing a prefetch never
// waits on an earlier load.
template <int BITS, int G, int D>
struct StepLoad {
    // value scale/zero pairs a lane stages: the groups of token l & 31 split
    // over lanes l and l + 32 when a token has 4 or 8 groups
    static constexpr int kVMG = D / G >= 4 ? D / G / 2 : D / G;
    static constexpr int kVW = (Geo<D>::kPV * BITS + 31) / 32;   // value code words per token
    uint32_t kw[2][Geo<D>::kKB];   // key code word of unit kb, token t0 + 16*blk + n
    typename MetaWords<Geo<D>::kKMC>::type ks, kz;   // key scale / zero of the lane's channels
    typename MetaWords<kVMG == 4 ? 4 : 2>::type vs, vz;   // value scale / zero, token t0 + (l & 31)
    uint32_t vw[8][kVW];    // value code words holding the lane's kPV channels, its 8 tokens
};

// The pair of a StepLoad field as floats: MB = 4 bytes (binary32) or 2
// (binary16, widened exactly).
template <int MB>
__device__ __forceinline__ float2 meta_pair(u32x2 v) {
    if constexpr (MB == 4) return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
    const half2_t h = as_h2(v.x);
    return make_float2(static_cast<float>(h[0]), static_cast<float>(h[1]));
}

template <int MB>
__device__ __forceinline__ float4 meta_quad(u32x4 v) {
    static_assert(MB == 4, "binary16 scale/zero are head_dim 128 only");
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// Token (within the step) of PV slot s for lane group q: the order in which
// QK^T leaves each lane its scores (rows 4q .. 4q+3 of both 16-token blocks).
__device__ __forceinline__ int pv_token(int q, int s) { return 16 * (s >> 2) + 4 * q + (s & 3); }


// ds is the store's head_dim: D itself, or (padded kernels) a multiple of
// 16 below D whose rows the lane geometry of D reads.  Lanes whose channels
// lie past ds load bytes of the next row or, past the slab's extent, zeros;
// the staging masks them.
template <int BITS, int G, int MB, int D, bool PAD>
__device__ __forceinline__ void issue_step(StepLoad<BITS, G, D>& L, const StoreView& S, const LaneOffsets& O,
                                           uint32_t t0, int n, int ds) {
    // a lane holding only channels past ds loads nothing (padded kernels)
    const auto lane_off = [](bool live, uint32_t off) { return (!PAD || live) ? off : kDeadOffset; };
    const uint32_t kRow = static_cast<uint32_t>(ds) * BITS / 8;   // code bytes per token
    constexpr int kMPT = D / G;                             // value groups per token of D's geometry
    constexpr int kKB = Geo<D>::kKB;
    constexpr int kKBytes = Geo<D>::kCPG * BITS / 8;        // a lane group's key code bytes: 4 .. 32
    const uint32_t ko = O.k + t0 * kRow;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        // the lane group's kCPG channels: one word per key unit (4-bit) or
        // per two units (2-bit)
        const uint32_t off = lane_off(O.k_live, ko + 16 * kRow * blk);
        uint32_t w[8];
        if constexpr (kKBytes >= 16) {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(S.kc, off, 0, kStreamLoad);
            w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
            if constexpr (kKBytes == 32) {
                const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(S.kc, off + 16, 0, kStreamLoad);
                w[4] = u.x; w[5] = u.y; w[6] = u.z; w[7] = u.w;
            }
        } else if constexpr (kKBytes == 8) {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(S.kc, off, 0, kStreamLoad);
            w[0] = t.x; w[1] = t.y;
        } else {
            w[0] = __builtin_amdgcn_raw_buffer_load_b32(S.kc, off, 0, kStreamLoad);
        }
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) L.kw[blk][kb] = w[BITS == 4 ? kb : kb / 2];
    }
    // key metadata of the step's group (a 32-token step never crosses one):
    // the lane's kKMC channels' pairs, kKMC * MB bytes
    const uint32_t kmo = lane_off(O.km_live, O.km + (t0 / G) * (static_cast<uint32_t>(ds) * MB));
    // value metadata: ceil(ds/G) pairs per token; the lane's groups
    const uint32_t vmo = O.vm + static_cast<uint32_t>((ds + G - 1) / G * MB) * t0;
    if constexpr (MB == 4) {
        if constexpr (Geo<D>::kKMC == 4) {
            L.ks = __builtin_amdgcn_raw_buffer_load_b128(S.ks, kmo, 0, kStreamLoad);
            L.kz = __builtin_amdgcn_raw_buffer_load_b128(S.kz, kmo, 0, kStreamLoad);
        } else {
            L.ks = __builtin_amdgcn_raw_buffer_load_b64(S.ks, kmo, 0, kStreamLoad);
            L.kz = __builtin_amdgcn_raw_buffer_load_b64(S.kz, kmo, 0, kStreamLoad);
        }
        if constexpr (kMPT == 1) {
            L.vs = u32x2{__builtin_amdgcn_raw_buffer_load_b32(S.vs, vmo, 0, kStreamLoad), 0u};
            L.vz = u32x2{__builtin_amdgcn_raw_buffer_load_b32(S.vz, vmo, 0, kStreamLoad), 0u};
        } else if constexpr (kMPT == 8) {
            L.vs = __builtin_amdgcn_raw_buffer_load_b128(S.vs, vmo, 0, kStreamLoad);
            L.vz = __builtin_amdgcn_raw_buffer_load_b128(S.vz, vmo, 0, kStreamLoad);
        } else {
            L.vs = __builtin_amdgcn_raw_buffer_load_b64(S.vs, vmo, 0, kStreamLoad);
            L.vz = __builtin_amdgcn_raw_buffer_load_b64(S.vz, vmo, 0, kStreamLoad);
        }
    } else {
        static_assert(D == 128, "binary16 scale/zero are head_dim 128 only");
        L.ks = u32x2{__builtin_amdgcn_raw_buffer_load_b32(S.ks, kmo, 0, kStreamLoad), 0u};
        L.kz = u32x2{__builtin_amdgcn_raw_buffer_load_b32(S.kz, kmo, 0, kStreamLoad), 0u};
        if constexpr (kMPT == 1) {
            L.vs = u32x2{static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(S.vs, vmo, 0, kStreamLoad)), 0u};
            L.vz = u32x2{static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(S.vz, vmo, 0, kStreamLoad)), 0u};
        } else {
            L.vs = u32x2{__builtin_amdgcn_raw_buffer_load_b32(S.vs, vmo, 0, kStreamLoad), 0u};
            L.vz = u32x2{__builtin_amdgcn_raw_buffer_load_b32(S.vz, vmo, 0, kStreamLoad), 0u};
        }
    }
    const uint32_t vo = O.v + t0 * kRow;
    // the lane's kPV channels start at bit kPV * n * BITS of the token row
    constexpr int kPV = Geo<D>::kPV;
    const uint32_t shift = (kPV * n * BITS) & 31;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const uint32_t off = lane_off(O.v_live, vo + (16 * (s >> 2) + (s & 3)) * kRow);
        if constexpr (StepLoad<BITS, G, D>::kVW == 2) {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(S.vc, off, 0, kStreamLoad);
            L.vw[s][0] = t.x; L.vw[s][1] = t.y;
        } else {
            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(S.vc, off, 0, kStreamLoad);
            // bring the lane's channels to the low bits
            L.vw[s][0] = (kPV * BITS >= 32) ? w : (w >> shift);
        }
    }
}

// Keeps the compiler from moving LDS accesses across this point.  The
// workgroup is one wave and a wave's LDS instructions execute in order, so
// no hardware barrier is needed between a lane's write and another lane's
// later read.
__device__ __forceinline__ void lds_order() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Rows are padded so that lanes reading different channel windows or groups
// in the same LDS cycle hit different banks.
constexpr int kKPad = 4;                      // floats of padding per 32 channels
constexpr int kVRow = kStep + 4;              // padded row of 32 tokens
__device__ __forceinline__ int kidx(int ch) { return ch + kKPad * (ch >> 5); }

template <int D>
struct Smem {
    alignas(16) float ks[D + kKPad * (D / 32)];       // key scale of the step's group
    alignas(16) float kz[D + kKPad * (D / 32)];       // key zero - M * scale
    alignas(16) float vs[D / kGroup][kVRow];          // value scale, [group][token]
    alignas(16) float vz[D / kGroup][kVRow];          // value zero - M * scale
    alignas(16) uint4 bq[D / 32][64];                 // QK^T B operand (queries), [unit][lane]
};

// The QK^T B operand of channel unit kb, kept in LDS rather than in 16
// registers across the step loop (the registers hold the prefetched loads).
template <int D>
__device__ __forceinline__ Frag query_frag(const Smem<D>& sm, int kb, int l) {
    const uint4 v = sm.bq[kb][l];
    Frag f;
    f.u[0] = v.x; f.u[1] = v.y; f.u[2] = v.z; f.u[3] = v.w;
    return f;
}

// Online-softmax state of one lane: head n, channel kPV (4q + r) + i in
// acc_o[i][r] (NPV = kPV accumulators).
template <int NPV>
struct SoftState {
    float m_run;
    float l_part;
    float4_t acc_o[NPV];
};

// The running max m only moves when a step's max exceeds it by more than
// kSlack (base 2), so most steps skip rescaling the accumulators; the
// unnormalized probabilities stay <= 2^kSlack = 256, exact enough in fp16
// (relative precision is unchanged) and far from its range limit.
constexpr float kSlack = 8.0f;

// Online softmax over one step's scores (base 2) and the PV B operand.
// Lane (q, n) holds head n's scores of step tokens 16*blk + 4q + r; with
// MASK, tokens at or past `limit` (step-relative) get probability 0.  The
// scale c2 = softmax_scale * log2(e) is positive, so the max is taken over
// the raw scores and scaled once.
// fp16: P is rounded to fp16 (relative 2^-11) and `lo` is unused.  bfloat16
// would lose 2^-9 that way, the largest error of the bfloat16 attend, so P
// is split: the high part is p with its low 16 bits cleared (a bfloat16,
// truncated), the low part the exact remainder rounded to bfloat16; PV
// takes one MFMA for each and P keeps 2^-16 relative.
template <bool MASK, bool BF, int NPV>
__device__ __forceinline__ Frag softmax_step(const float4_t (&acc_s)[2], SoftState<NPV>& st, float c2,
                                             int limit, int q, Frag& lo) {
    float sv[8];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sc = acc_s[blk][r];
            if constexpr (MASK) sc = (16 * blk + 4 * q + r) < limit ? sc : -INFINITY;
            sv[4 * blk + r] = sc;
        }
    float mloc = sv[0];
#pragma unroll
    for (int s = 1; s < 8; ++s) mloc = __builtin_elementwise_maximum(mloc, sv[s]);
    const float m_step = rows_max(mloc) * c2;
    const float m_new = m_step > st.m_run + kSlack ? m_step : st.m_run;
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);   // 1 when m did not move
    st.m_run = m_new;
#pragma unroll
    for (int s = 0; s < 8; ++s) sv[s] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[s], c2, -m_new));
    float psum = sv[0];
#pragma unroll
    for (int s = 1; s < 8; ++s) psum += sv[s];
    st.l_part = __builtin_fmaf(st.l_part, alpha, psum);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int i = 0; i < NPV; ++i) st.acc_o[i] *= alpha;
    }
    Frag bp;                                  // P^T, slot s <-> step token pv_token(q, s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (BF) {
            const uint32_t u0 = __float_as_uint(sv[2 * j]), u1 = __float_as_uint(sv[2 * j + 1]);
            bp.u[j] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);        // high halves
            lo.u[j] = bf16_pair(sv[2 * j] - __uint_as_float(u0 & 0xffff0000u),
                                sv[2 * j + 1] - __uint_as_float(u1 & 0xffff0000u));
        } else {
            half2_t h;
            h[0] = static_cast<_Float16>(sv[2 * j]);
            h[1] = static_cast<_Float16>(sv[2 * j + 1]);
            bp.u[j] = as_u32(h);
        }
    }
    return bp;
}

template <bool BF, int NPV>
__device__ __forceinline__ Frag softmax_any(const float4_t (&acc_s)[2], SoftState<NPV>& st, float c2,
                                            int limit, int q, Frag& lo) {
    if (limit >= kStep) return softmax_step<false, BF>(acc_s, st, c2, limit, q, lo);
    return softmax_step<true, BF>(acc_s, st, c2, limit, q, lo);
}

// One step of store tokens [t0, t0 + 32), tokens at or past n_quant masked.
// PAD: the store's head_dim ds is below D; the key scale and zero of
// channels at or past ds are staged as 0, so those channels of K are exactly
// 0 whatever their codes (the query is 0 there too), and the value channels
// past ds only reach outputs that are never stored.
template <int BITS, int G, int MB, bool BF, int D, bool PAD>
__device__ __forceinline__ void store_step(const StepLoad<BITS, G, D>& L, Smem<D>& sm,
                                           SoftState<Geo<D>::kPV>& st, int t0, int n_quant, float c2,
                                           int l, int n, int q, int ds) {
    // ---- stage this step's metadata in LDS (zero' = zero - M * scale')
    constexpr float kM = kCodeOffset<BITS, BF>;
    constexpr int kMPT = D / G;                 // value groups per token
    constexpr int kCPG = Geo<D>::kCPG, kKB = Geo<D>::kKB, kPV = Geo<D>::kPV;
    lds_order();
    if constexpr (Geo<D>::kKMC == 4) {
        // channels 4l .. 4l + 3; key scale times 2^-e of each channel's code
        // position (code_pairs)
        float4 ks = meta_quad<MB>(L.ks), kz = meta_quad<MB>(L.kz);
        if constexpr (PAD) {
            if (4 * l >= ds) ks = kz = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        const float sc[4] = {ks.x, ks.y, ks.z, ks.w}, zc[4] = {kz.x, kz.y, kz.z, kz.w};
        float so[4], zo[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            so[c] = sc[c] * kscale_factor<BITS, BF>(4 * l + c);
            zo[c] = __builtin_fmaf(-kM, so[c], zc[c]);
        }
        *reinterpret_cast<float4*>(&sm.ks[kidx(4 * l)]) = make_float4(so[0], so[1], so[2], so[3]);
        *reinterpret_cast<float4*>(&sm.kz[kidx(4 * l)]) = make_float4(zo[0], zo[1], zo[2], zo[3]);
    } else if (2 * l < D) {
        // key scale times 2^-e of its channel's code position (code_pairs)
        float2 ks = meta_pair<MB>(L.ks), kz = meta_pair<MB>(L.kz);
        if constexpr (PAD) {
            if (2 * l >= ds) ks = kz = make_float2(0.0f, 0.0f);
        }
        const float s0 = ks.x * kscale_factor<BITS, BF>(2 * l);
        const float s1 = ks.y * kscale_factor<BITS, BF>(2 * l + 1);
        *reinterpret_cast<float2*>(&sm.ks[kidx(2 * l)]) = make_float2(s0, s1);
        *reinterpret_cast<float2*>(&sm.kz[kidx(2 * l)]) =
            make_float2(__builtin_fmaf(-kM, s0, kz.x), __builtin_fmaf(-kM, s1, kz.y));
    }
    if constexpr (kMPT == 8) {
        // token l & 31, groups 4 (l >> 5) .. 4 (l >> 5) + 3
        const float4 vs = meta_quad<MB>(L.vs), vz = meta_quad<MB>(L.vz);
        const float sv[4] = {vs.x, vs.y, vs.z, vs.w}, zv[4] = {vz.x, vz.y, vz.z, vz.w};
        const int tt = l & 31, gg = (l >> 5) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            sm.vs[gg + c][tt] = sv[c];
            sm.vz[gg + c][tt] = __builtin_fmaf(-kM, sv[c], zv[c]);
        }
    } else {
        // lanes l and l + 32 hold the same token; with 2 groups or 1 per
        // token they hold the same groups too and write the same values
        const float2 vs = meta_pair<MB>(L.vs), vz = meta_pair<MB>(L.vz);
        const int tt = l & 31;
        const int gg = kMPT == 4 ? (l >> 5) * 2 : 0;
        sm.vs[gg][tt] = vs.x;
        sm.vz[gg][tt] = __builtin_fmaf(-kM, vs.x, vz.x);
        if constexpr (kMPT != 1) {
            sm.vs[gg + 1][tt] = vs.y;
            sm.vz[gg + 1][tt] = __builtin_fmaf(-kM, vs.y, vz.y);
        }
    }
    lds_order();

    // ---- S^T = K Q^T, token t0 + 16*blk + n, channel unit kb of group q
    float4_t acc_s[2] = {float4_t{0.0f, 0.0f, 0.0f, 0.0f}, float4_t{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
        const int cb = kidx(kCPG * q + 8 * kb);
        const float4 s0 = *reinterpret_cast<const float4*>(&sm.ks[cb]);
        const float4 s1 = *reinterpret_cast<const float4*>(&sm.ks[cb + 4]);
        const float4 z0 = *reinterpret_cast<const float4*>(&sm.kz[cb]);
        const float4 z1 = *reinterpret_cast<const float4*>(&sm.kz[cb + 4]);
        const float sl[4] = {s0.x, s0.y, s0.z, s0.w}, sh[4] = {s1.x, s1.y, s1.z, s1.w};
        const float zl[4] = {z0.x, z0.y, z0.z, z0.w}, zh[4] = {z1.x, z1.y, z1.z, z1.w};
        const Frag bq = query_frag(sm, kb, l);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            Frag ka;
            if constexpr (kByteCodes<BITS, BF>) {
                // channels (2j, 2j+1) of the unit: byte j of the even and odd nibbles
                uint32_t lo, hi;
                split_nibbles(L.kw[blk][kb], lo, hi);
                const float sc[8] = {sl[0], sl[1], sl[2], sl[3], sh[0], sh[1], sh[2], sh[3]};
                const float zc[8] = {zl[0], zl[1], zl[2], zl[3], zh[0], zh[1], zh[2], zh[3]};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ka.u[j] = bf16_pair(__builtin_fmaf(byte_f32(lo, j), sc[2 * j], zc[2 * j]),
                                        __builtin_fmaf(byte_f32(hi, j), sc[2 * j + 1], zc[2 * j + 1]));
            } else {
                uint32_t pr[4];
                code_pairs<BITS, BF>(L.kw[blk][kb], kb & 1, pr);
#pragma unroll
                for (int j = 0; j < 4; ++j) ka.u[j] = deq2<BF>(pr[j], sl[j], zl[j], sh[j], zh[j]);
            }
            acc_s[blk] = mfma<BF>(ka, bq, acc_s[blk]);
        }
    }

    Frag bp_lo;
    const Frag bp = softmax_any<BF>(acc_s, st, c2, n_quant - t0, q, bp_lo);

    // ---- O^T += V^T P^T: MFMA i covers channels kPV*m + i, m = 0..15.  Slot s
    // of lane (q, m) is channel kPV*m + i of step token pv_token(q, s).
    const int vg = (kPV * n) / G;               // value group of the lane's kPV channels
    const float4 vsa = *reinterpret_cast<const float4*>(&sm.vs[vg][4 * q]);
    const float4 vsb = *reinterpret_cast<const float4*>(&sm.vs[vg][16 + 4 * q]);
    const float4 vza = *reinterpret_cast<const float4*>(&sm.vz[vg][4 * q]);
    const float4 vzb = *reinterpret_cast<const float4*>(&sm.vz[vg][16 + 4 * q]);
    const float vsc[8] = {vsa.x, vsa.y, vsa.z, vsa.w, vsb.x, vsb.y, vsb.z, vsb.w};
    const float vzp[8] = {vza.x, vza.y, vza.z, vza.w, vzb.x, vzb.y, vzb.z, vzb.w};
    if constexpr (kByteCodes<BITS, BF>) {
        // token slot s: the even channels' codes in the bytes of vlo, the odd
        // ones' in vhi; channel i of the lane's kPV is byte i/2 of one of them
        constexpr int kVW = StepLoad<BITS, G, D>::kVW;
        uint32_t vlo[8][kVW], vhi[8][kVW];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int w = 0; w < kVW; ++w) split_nibbles(L.vw[t][w], vlo[t][w], vhi[t][w]);
#pragma unroll
        for (int i = 0; i < kPV; ++i) {
            const int wi = i >> 3, ii = i & 7;          // word and place of channel i
            Frag va;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w0 = (ii & 1) ? vhi[2 * j][wi] : vlo[2 * j][wi];
                const uint32_t w1 = (ii & 1) ? vhi[2 * j + 1][wi] : vlo[2 * j + 1][wi];
                va.u[j] = bf16_pair(__builtin_fmaf(byte_f32(w0, ii >> 1), vsc[2 * j], vzp[2 * j]),
                                    __builtin_fmaf(byte_f32(w1, ii >> 1), vsc[2 * j + 1], vzp[2 * j + 1]));
            }
            st.acc_o[i] = mfma<BF>(va, bp, st.acc_o[i]);
            st.acc_o[i] = mfma<BF>(va, bp_lo, st.acc_o[i]);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kPV; ++i) {
        // code of channel i of the lane's kPV: word wi, field ii (4-bit:
        // nibble ii; 2-bit: two-bit field ii)
        constexpr uint32_t kMask = BITS == 4 ? 0x000F000Fu : 0x00030003u;
        constexpr int kCPW = 32 / BITS;
        const int wi = i / kCPW, ii = i % kCPW;
        const uint32_t byte = BITS == 4 ? (ii >> 1) : (ii >> 2);
        const uint32_t shift = BITS == 4 ? 4 * (ii & 1) : 2 * (ii & 3);
        const uint32_t sel = 0x0C000C00u | ((4u + byte) << 16) | byte;
        Frag va;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t x = __builtin_amdgcn_perm(L.vw[2 * j + 1][wi], L.vw[2 * j][wi], sel);
            const uint32_t pr = and_or(x >> shift, kMask, kMagic<BF>);
            va.u[j] = deq2<BF>(pr, vsc[2 * j], vzp[2 * j], vsc[2 * j + 1], vzp[2 * j + 1]);
        }
        st.acc_o[i] = mfma<BF>(va, bp, st.acc_o[i]);
        if constexpr (BF) st.acc_o[i] = mfma<BF>(va, bp_lo, st.acc_o[i]);
    }
}

// One step of fp16 residual tokens [t0, t0 + 32), tokens at or past n_res masked.
// Residual token i of the slab is row (head + i) mod ring (head < ring).
__device__ __forceinline__ int ring_row(int tok, int head, int ring) {
    const int r = tok + head;
    return r >= ring ? r - ring : r;
}

// Rows have ds channels (PAD: ds < D); channels at or past ds are not
// loaded and read as 0 (ds is a multiple of 16, so every 8- or 4-channel
// load is wholly inside a row or wholly past it).
// Token new_tok (a fused append; -1 if none) is read from the rows knew /
// vnew instead of the window.
template <int BITS, bool BF, int D, bool PAD>
__device__ __forceinline__ void residual_step(const uint16_t* kr, const uint16_t* vr, const Smem<D>& sm,
                                              SoftState<Geo<D>::kPV>& st, int t0, int n_res, float c2,
                                              int l, int n, int q, int head, int ring, int ds,
                                              int new_tok, const uint16_t* knew, const uint16_t* vnew) {
    constexpr int kCPG = Geo<D>::kCPG, kKB = Geo<D>::kKB, kPV = Geo<D>::kPV;
    const int last = n_res - 1;
    const auto krow = [&](int tok) { return tok == new_tok ? knew : kr + ring_row(tok, head, ring) * ds; };
    const auto vrow = [&](int tok) { return tok == new_tok ? vnew : vr + ring_row(tok, head, ring) * ds; };
    // Every row of the step is loaded up front (K rows of both 16-token
    // blocks and the V rows), so a residual step costs one memory round trip.
    uint32_t rn[2][kCPG / 2];                   // the lane group's key channels, natural order
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const uint4* src = reinterpret_cast<const uint4*>(krow(min(t0 + 16 * blk + n, last)) + kCPG * q);
#pragma unroll
        for (int v = 0; v < kCPG / 8; ++v) {
            const uint4 t = (!PAD || kCPG * q + 8 * v < ds) ? src[v] : make_uint4(0u, 0u, 0u, 0u);
            rn[blk][4 * v] = t.x; rn[blk][4 * v + 1] = t.y; rn[blk][4 * v + 2] = t.z; rn[blk][4 * v + 3] = t.w;
        }
    }
    // V rows: lane (q, m=n) takes channels kPV*n .. kPV*n + kPV - 1 of its 8 tokens
    uint32_t vw[8][kPV / 2];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const uint16_t* p = vrow(min(t0 + pv_token(q, s), last)) + kPV * n;
        if constexpr (kPV >= 8) {
#pragma unroll
            for (int v = 0; v < kPV / 8; ++v) {
                const uint4 t = (!PAD || kPV * n + 8 * v < ds) ? reinterpret_cast<const uint4*>(p)[v]
                                                               : make_uint4(0u, 0u, 0u, 0u);
                vw[s][4 * v] = t.x; vw[s][4 * v + 1] = t.y; vw[s][4 * v + 2] = t.z; vw[s][4 * v + 3] = t.w;
            }
        } else {
            const uint2 t = (!PAD || kPV * n < ds) ? *reinterpret_cast<const uint2*>(p) : make_uint2(0u, 0u);
            vw[s][0] = t.x; vw[s][1] = t.y;
        }
    }
    float4_t acc_s[2] = {float4_t{0.0f, 0.0f, 0.0f, 0.0f}, float4_t{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            Frag ka;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (kByteCodes<BITS, BF>) {
                    ka.u[j] = rn[blk][4 * kb + j];        // natural order: channels 8kb + 2j, + 1
                } else {
                    const int c0 = 8 * kb + j, c1 = 8 * kb + j + 4;
                    const uint32_t s0 = (c0 & 1) ? 0x0302u : 0x0100u;
                    const uint32_t s1 = (c1 & 1) ? 0x0706u : 0x0504u;
                    ka.u[j] = __builtin_amdgcn_perm(rn[blk][c1 >> 1], rn[blk][c0 >> 1], (s1 << 16) | s0);
                }
            }
            acc_s[blk] = mfma<BF>(ka, query_frag(sm, kb, l), acc_s[blk]);
        }
    }
    Frag bp_lo;
    const Frag bp = softmax_any<BF>(acc_s, st, c2, n_res - t0, q, bp_lo);
#pragma unroll
    for (int i = 0; i < kPV; ++i) {
        Frag va;
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int j = 0; j < 4; ++j) va.u[j] = __builtin_amdgcn_perm(vw[2 * j + 1][i >> 1], vw[2 * j][i >> 1], sel);
        st.acc_o[i] = mfma<BF>(va, bp, st.acc_o[i]);
        if constexpr (BF) st.acc_o[i] = mfma<BF>(va, bp_lo, st.acc_o[i]);
    }
}

// One wave: sequence b, kv head kv, one split.  The token axis of a slab is
// the store tokens [0, n_quant) in steps_q 32-token steps followed by the
// residual tokens [0, n_res); split s covers the steps [s*spw, (s+1)*spw) of
// that axis, so one wave may finish the store and start the residual.
// Offsets within a slab fit in 32 bits: the ABI keeps n_quant and n_res
// below 2^24 tokens.
// Head_dim 256 doubles every per-lane array (16 PV accumulators, 64 key
// channels per lane group) and runs at 2 waves per SIMD (fp16, two buffers)
// or 1 (bfloat16, three buffers: its dequantization needs the registers).
#ifndef KIVI_ATTEND_BF16_D256_WAVES
#define KIVI_ATTEND_BF16_D256_WAVES 1
#endif
#ifndef KIVI_ATTEND_BF16_D256_NBUF
#define KIVI_ATTEND_BF16_D256_NBUF 3
#endif
template <bool BF, int D> constexpr int kWavesPerSimd =
    (BF && D == 256) ? KIVI_ATTEND_BF16_D256_WAVES : D == 256 ? 2 : BF ? KIVI_ATTEND_BF16_WAVES
                                                                    : KIVI_ATTEND_WAVES_PER_SIMD;
template <bool BF, int D> constexpr int kNBufOf = (BF && D == 256) ? KIVI_ATTEND_BF16_D256_NBUF : D == 256 ? 2 : kNBuf;

// PAD: the stores, q, the residual rows and the partials have ds =
// a.head_dim channels, a multiple of 16 below D, and the lanes of D's
// geometry past ds compute on zeros (see store_step and residual_step).
template <int BITS, int GQA, int G, int MB, bool BF, int D, bool PAD>
__device__ __forceinline__ void partial_body(const AttendArgs& a, int spw, int steps_q, int64_t n_split,
                                             float* __restrict__ ws_o, float* __restrict__ ws_ml)
{
    constexpr int kCPG = Geo<D>::kCPG, kKB = Geo<D>::kKB, kPV = Geo<D>::kPV;
    const int ds = PAD ? a.head_dim : D;
    __shared__ Smem<D> sm;
    const int l = threadIdx.x;
    const int n = l & 15;
    const int q = l >> 4;
    const int split = blockIdx.x;
    const int64_t bkv = blockIdx.y;
    const int64_t b = bkv / a.Hkv;
    const int kv = static_cast<int>(bkv - b * a.Hkv);
    const int64_t qrow0 = b * a.Hq + static_cast<int64_t>(kv) * GQA;

    // Token counts of this sequence: the uniform bounds, or the per-sequence
    // lengths clamped to them (so no load can leave the bounded slab).
    int nq = static_cast<int>(a.n_quant);
    int nr = static_cast<int>(a.n_res);
    if (a.seq_n_quant) {
        nq = min(max(a.seq_n_quant[b], 0), nq);
        nr = min(max(a.seq_n_res[b], 0), nr);
    }
    const int s0 = split * spw, s1 = s0 + spw;
    const int j0 = s0 * kStep;                                  // store tokens [j0, j1)
    const int j1 = min(min(s1, steps_q) * kStep, nq);
    const int r0 = max(s0 - steps_q, 0) * kStep;                // residual tokens [r0, r1)
    const int r1 = min(max(s1 - steps_q, 0) * kStep, nr);
    const bool has_store = j0 < j1;

    // Store part: buffer views and the first kNB - 1 steps' loads, issued
    // before the query so the two HBM latencies overlap.
    const int words = ds * BITS / 32;                   // code words per token
    constexpr int kMetaPerTok = D / G;                  // value groups per token of D's geometry
    const int meta_per_tok = (ds + G - 1) / G;          // ... and of the store
    constexpr int kNB = kNBufOf<BF, D>;
    StoreView S;
    LaneOffsets O;
    StepLoad<BITS, G, D> buf[kNB];
    // Every prefetch is issued, also past the split's end (to a token far
    // outside the buffers' extent, which the buffer unit answers with zeros
    // and no memory access): a conditional issue makes the compiler wait for
    // all outstanding loads at the join.
    const auto pref = [j1](int t) { return t < j1 ? static_cast<uint32_t>(t) : kFarToken; };
    if (has_store) {
        const uint32_t n_groups = static_cast<uint32_t>((nq + G - 1) / G);
        S.kc = make_rsrc(a.k_codes + bkv * a.k_codes_bh_stride, static_cast<uint32_t>(nq) * words * 4u);
        const char* kmeta_s = static_cast<const char*>(a.k_scale) + bkv * a.k_meta_bh_stride * MB;
        const char* kmeta_z = static_cast<const char*>(a.k_zero) + bkv * a.k_meta_bh_stride * MB;
        const char* vmeta_s = static_cast<const char*>(a.v_scale) + bkv * a.v_meta_bh_stride * MB;
        const char* vmeta_z = static_cast<const char*>(a.v_zero) + bkv * a.v_meta_bh_stride * MB;
        S.ks = make_rsrc(kmeta_s, n_groups * ds * MB);
        S.kz = make_rsrc(kmeta_z, n_groups * ds * MB);
        S.vc = make_rsrc(a.v_codes + bkv * a.v_codes_bh_stride, static_cast<uint32_t>(nq) * words * 4u);
        S.vs = make_rsrc(vmeta_s, static_cast<uint32_t>(nq) * meta_per_tok * MB);
        S.vz = make_rsrc(vmeta_z, static_cast<uint32_t>(nq) * meta_per_tok * MB);
        // the lane group's channels start at word kCPG * q * BITS / 32 of a
        // token row; the lane's PV channels at word kPV * n * BITS / 32
        O.k = static_cast<uint32_t>(n * words + kCPG * q * BITS / 32) * 4u;
        O.v = static_cast<uint32_t>(4 * q * words + kPV * n * BITS / 32) * 4u;
        // lanes past D / kKMC load but stage nothing
        O.km = static_cast<uint32_t>(l) * (Geo<D>::kKMC * MB);
        O.vm = kMetaPerTok >= 4
                   ? static_cast<uint32_t>(l & 31) * (meta_per_tok * MB) +
                         static_cast<uint32_t>(l >> 5) * (kMetaPerTok / 2 * MB)
                   : static_cast<uint32_t>(l & 31) * (meta_per_tok * MB);
        if constexpr (PAD) {
            O.k_live = kCPG * q < ds;
            O.v_live = kPV * n < ds;
            O.km_live = Geo<D>::kKMC * l < ds;
        }
#pragma unroll
        for (int u = 0; u + 1 < kNB; ++u) issue_step<BITS, G, MB, D, PAD>(buf[u], S, O, pref(j0 + u * kStep), n, ds);
    }

    // B operand of QK^T: q of head n (zero for n >= GQA) in slot order.
    {
        Frag bq[kKB];
        uint32_t qn[kCPG / 2];                // channels kCPG*q .. kCPG*q + kCPG - 1, natural order
        if (n < GQA) {
            const uint4* src = reinterpret_cast<const uint4*>(a.q + (qrow0 + n) * ds + kCPG * q);
#pragma unroll
            for (int v = 0; v < kCPG / 8; ++v) {
                const uint4 t = (!PAD || kCPG * q + 8 * v < ds) ? src[v] : make_uint4(0u, 0u, 0u, 0u);
                qn[4 * v] = t.x; qn[4 * v + 1] = t.y; qn[4 * v + 2] = t.z; qn[4 * v + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < kCPG / 2; ++v) qn[v] = 0u;
        }
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (kByteCodes<BITS, BF>) {
                    // slots (2j, 2j+1) = channels (8kb + 2j, 8kb + 2j + 1)
                    bq[kb].u[j] = qn[4 * kb + j];
                } else {
                    // slots (2j, 2j+1) = channels (8kb + j, 8kb + j + 4) of the lane's window
                    const int c0 = 8 * kb + j, c1 = 8 * kb + j + 4;
                    const uint32_t s0 = (c0 & 1) ? 0x0302u : 0x0100u;
                    const uint32_t s1 = (c1 & 1) ? 0x0706u : 0x0504u;
                    bq[kb].u[j] = __builtin_amdgcn_perm(qn[c1 >> 1], qn[c0 >> 1], (s1 << 16) | s0);
                }
            }
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) sm.bq[kb][l] = make_uint4(bq[kb].u[0], bq[kb].u[1], bq[kb].u[2], bq[kb].u[3]);
        lds_order();
    }

    const float c2 = a.softmax_scale * kLog2e;
    SoftState<kPV> st;
    st.m_run = -INFINITY;
    st.l_part = 0.0f;
#pragma unroll
    for (int i = 0; i < kPV; ++i) st.acc_o[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    if (has_store) {
        // kNB buffers in rotation: while step t computes, the loads of the
        // next kNB - 1 steps are in flight.
        for (int t0 = j0; t0 < j1; t0 += kNB * kStep) {
#pragma unroll
            for (int u = 0; u < kNB; ++u) {
                issue_step<BITS, G, MB, D, PAD>(buf[(u + kNB - 1) % kNB], S, O, pref(t0 + (u + kNB - 1) * kStep), n, ds);
                store_step<BITS, G, MB, BF, D, PAD>(buf[u], sm, st, t0 + u * kStep, j1, c2, l, n, q, ds);
                if (t0 + (u + 1) * kStep >= j1) goto store_done;
            }
        }
    store_done:;
    }
    if (r0 < r1) {
        const uint16_t* kr = a.k_res + bkv * a.res_bh_stride;
        const uint16_t* vr = a.v_res + bkv * a.res_bh_stride;
        // a fused append's token: the last of the window (uniform batches only)
        const int new_tok = a.k_new ? nr - 1 : -1;
        const uint16_t* knew = a.k_new ? a.k_new + bkv * ds : kr;
        const uint16_t* vnew = a.k_new ? a.v_new + bkv * ds : vr;
        for (int t0 = r0; t0 < r1; t0 += kStep)
            residual_step<BITS, BF, D, PAD>(kr, vr, sm, st, t0, r1, c2, l, n, q, a.res_head, a.res_ring, ds,
                                            new_tok, knew, vnew);
        if (a.k_new && r1 == nr) {
            // this wave holds the new token: it writes the token's K and V
            // rows into the window's row new_row (ds / 8 lanes of 16 bytes
            // each), which no other wave of this launch reads
            const int chunks = ds / 8;
            if (l < 2 * chunks) {
                const bool val = l >= chunks;
                const int c = val ? l - chunks : l;
                const uint4 row = *reinterpret_cast<const uint4*>((val ? vnew : knew) + c * 8);
                uint16_t* dst = const_cast<uint16_t*>(val ? vr : kr) + a.new_row * ds + c * 8;
                *reinterpret_cast<uint4*>(dst) = row;
            }
        }
    }

    // ---- partial (m, l, o) of head n: lane (q, n) holds channels
    // kPV * (4q + r) + i (= kCPG q + kPV r + i)
    const float l_tot = rows_sum(st.l_part);
    if (n < GQA) {
        float* dst = ws_o + ((qrow0 + n) * n_split + split) * ds + kCPG * q;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < kPV / 4; ++c)
                if (!PAD || kCPG * q + kPV * r + 4 * c < ds)
                    *reinterpret_cast<float4*>(dst + kPV * r + 4 * c) =
                        make_float4(st.acc_o[4 * c][r], st.acc_o[4 * c + 1][r], st.acc_o[4 * c + 2][r],
                                    st.acc_o[4 * c + 3][r]);
        if (q == 0) {
            float* ml = ws_ml + ((qrow0 + n) * n_split + split) * 2;
            ml[0] = st.m_run;
            ml[1] = l_tot;
        }
    }
}

template <int BITS, int GQA, int G, int MB, bool BF, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<BF, D>))) void attend_partial_kernel(const AttendArgs a, int spw, int steps_q,
                                                            int64_t n_split, float* __restrict__ ws_o,
                                                            float* __restrict__ ws_ml)
{
    partial_body<BITS, GQA, G, MB, BF, D, false>(a, spw, steps_q, n_split, ws_o, ws_ml);
}

// Store head_dims below D that are not 64 or 128 (multiples of 16, groups
// of 32, binary32 scale/zero) on D's geometry: 16 .. 48 on 64, 80 .. 112 on
// 128, 144 .. 240 on 256.
template <int BITS, int GQA, bool BF, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<BF, D>))) void attend_partial_padded_kernel(const AttendArgs a, int spw, int steps_q,
                                                            int64_t n_split, float* __restrict__ ws_o,
                                                            float* __restrict__ ws_ml)
{
    partial_body<BITS, GQA, kGroup, 4, BF, D, true>(a, spw, steps_q, n_split, ws_o, ws_ml);
}

// ---------------------------------------------------------------------------
// Host side: launch the partial kernel of one instantiation, and the dispatch
// over (bits, group size, query heads per kv head) for one metadata width
// MB and element format BF.  Each translation unit that calls
// launch_partials instantiates its own set of kernels.
// ---------------------------------------------------------------------------
template <int BITS, int GQA, int G, int MB, bool BF, int D>
hipError_t launch_partial(const AttendArgs& a, const AttendPlan& p, float* ws_o, float* ws_ml,
                          hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(p.n_split), static_cast<uint32_t>(a.B * a.Hkv));
    hipLaunchKernelGGL((attend_partial_kernel<BITS, GQA, G, MB, BF, D>), grid, dim3(64), 0, stream, a,
                       static_cast<int>(p.steps_per_wave), static_cast<int>(p.steps_q), p.n_split,
                       ws_o, ws_ml);
    return hipGetLastError();
}

template <int BITS, int G, int MB, bool BF, int D = 128>
hipError_t launch_partial_gqa(const AttendArgs& a, const AttendPlan& p, float* ws_o, float* ws_ml,
                              hipStream_t stream) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_partial<BITS, 1, G, MB, BF, D>(a, p, ws_o, ws_ml, stream);
        case 2: return launch_partial<BITS, 2, G, MB, BF, D>(a, p, ws_o, ws_ml, stream);
        case 4: return launch_partial<BITS, 4, G, MB, BF, D>(a, p, ws_o, ws_ml, stream);
        default: return launch_partial<BITS, 8, G, MB, BF, D>(a, p, ws_o, ws_ml, stream);
    }
}

template <int MB, bool BF>
hipError_t launch_partials(const AttendArgs& a, const AttendPlan& p, float* ws_o, float* ws_ml,
                           hipStream_t stream) {
    const bool four = a.bits == 4;
    if constexpr (MB == 4) {
        // head_dim 64 and 256 (groups of 32, binary32 scale/zero)
        if (a.head_dim == 64)
            return four ? launch_partial_gqa<4, 32, MB, BF, 64>(a, p, ws_o, ws_ml, stream)
                        : launch_partial_gqa<2, 32, MB, BF, 64>(a, p, ws_o, ws_ml, stream);
        if (a.head_dim == 256)
            return four ? launch_partial_gqa<4, 32, MB, BF, 256>(a, p, ws_o, ws_ml, stream)
                        : launch_partial_gqa<2, 32, MB, BF, 256>(a, p, ws_o, ws_ml, stream);
    }
    switch (a.group) {
        case 64: return four ? launch_partial_gqa<4, 64, MB, BF>(a, p, ws_o, ws_ml, stream)
                             : launch_partial_gqa<2, 64, MB, BF>(a, p, ws_o, ws_ml, stream);
        case 128: return four ? launch_partial_gqa<4, 128, MB, BF>(a, p, ws_o, ws_ml, stream)
                              : launch_partial_gqa<2, 128, MB, BF>(a, p, ws_o, ws_ml, stream);
        default: return four ? launch_partial_gqa<4, 32, MB, BF>(a, p, ws_o, ws_ml, stream)
                             : launch_partial_gqa<2, 32, MB, BF>(a, p, ws_o, ws_ml, stream);
    }
}

// The bfloat16 partials (binary32 scale/zero), compiled in attend_bf16.hip.
hipError_t launch_attend_partial_bf16(const AttendArgs& a, const AttendPlan& p, float* ws_o,
                                      float* ws_ml, hipStream_t stream);

// The padded partial kernels: a store head_dim ds that is not 64, 128 or
// 256 runs on the geometry of the next of them (groups of 32, binary32
// scale/zero).
template <int BITS, int GQA, bool BF, int D>
hipError_t launch_padded(const AttendArgs& a, const AttendPlan& p, float* ws_o, float* ws_ml,
                         hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(p.n_split), static_cast<uint32_t>(a.B * a.Hkv));
    hipLaunchKernelGGL((attend_partial_padded_kernel<BITS, GQA, BF, D>), grid, dim3(64), 0, stream, a,
                       static_cast<int>(p.steps_per_wave), static_cast<int>(p.steps_q), p.n_split,
                       ws_o, ws_ml);
    return hipGetLastError();
}

template <int BITS, bool BF, int D>
hipError_t launch_padded_gqa(const AttendArgs& a, const AttendPlan& p, float* ws_o, float* ws_ml,
                             hipStream_t stream) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_padded<BITS, 1, BF, D>(a, p, ws_o, ws_ml, stream);
        case 2: return launch_padded<BITS, 2, BF, D>(a, p, ws_o, ws_ml, stream);
        case 4: return launch_padded<BITS, 4, BF, D>(a, p, ws_o, ws_ml, stream);
        default: return launch_padded<BITS, 8, BF, D>(a, p, ws_o, ws_ml, stream);
    }
}

template <bool BF>
hipError_t launch_partials_padded(const AttendArgs& a, const AttendPlan& p, float* ws_o, float* ws_ml,
                                  hipStream_t stream) {
    const bool four = a.bits == 4;
    if (a.head_dim < 64)
        return four ? launch_padded_gqa<4, BF, 64>(a, p, ws_o, ws_ml, stream)
                    : launch_padded_gqa<2, BF, 64>(a, p, ws_o, ws_ml, stream);
    if (a.head_dim < 128)
        return four ? launch_padded_gqa<4, BF, 128>(a, p, ws_o, ws_ml, stream)
                    : launch_padded_gqa<2, BF, 128>(a, p, ws_o, ws_ml, stream);
    return four ? launch_padded_gqa<4, BF, 256>(a, p, ws_o, ws_ml, stream)
                : launch_padded_gqa<2, BF, 256>(a, p, ws_o, ws_ml, stream);
}

// Compiled in attend_pad.hip (fp16, which hands bfloat16 calls to the
// second) and attend_pad_bf16.hip.
hipError_t launch_attend_partial_padded(const AttendArgs& a, const AttendPlan& p, float* ws_o,
                                        float* ws_ml, hipStream_t stream);
hipError_t launch_attend_partial_padded_bf16(const AttendArgs& a, const AttendPlan& p, float* ws_o,
                                             float* ws_ml, hipStream_t stream);

}  // namespace kivi
