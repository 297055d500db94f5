// flush.hip -- the KIVI flush kernels for gfx950: per-channel keys and
// per-token values, quantized to 2 or 4 bits, codes bit-packed into uint32,
// one scale and zero per group (binary32, or binary16 for fp16 caches),
// optional fused fp16 reconstruction.
//
// Sources, cited by page title and section:
//   [Metal post] blog post "A 5.65x Metal Kernel That Made My LLM Exactly 0%
//                Faster": "What we're actually optimizing" (the quantizer),
//                "The layout problem that shapes everything", "Kernel A",
//                "Kernel B", "Three ways to be off by one bit".
//
// Both kernels give one wave one tile of tokens x 128 channels with the lane
// mapping of kivi_device.h.  For keys the tile is exactly one token group of
// every channel (G = 32, 64 or 128 tokens), so a lane's G/4 tokens x 8
// channels cover a quarter of each of its 8 channel groups; the four
// quarters meet with two cross-row exchanges and no LDS.  For values the
// tile is 32 tokens and each token row's 128 channels are groups of G
// channels, i.e. G/8 lanes of 8; two quad exchanges finish a group of 32,
// a half-row mirror one of 64 and a row mirror one of 128.  The
// Metal kernels used a thread per strided key group and a 32-lane SIMD-group
// per value group; on wave64 both layouts read the same coalesced tile.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

// ---------------------------------------------------------------------------
// Keys: group = (bh, token group g, channel d) over tokens [32g, min(32g+32, S))
// ---------------------------------------------------------------------------
// Key rows.  Where head_dim/8 is not a power of two, a row of exactly
// head_dim/8 lanes can fit more tokens in a wave than RowGeo's padded rows;
// it is taken where that needs fewer passes over a group of 32 tokens
// (head_dims 80, 96, 144 and 160: 6, 7, 11 and 11 passes instead of 8, 8, 16
// and 16), and the rows' per-channel min/max then meet through the wave's LDS
// instead of lane exchanges.  Measured on MI355X (4-bit keys, 32768 tokens
// per slab, one flush), fp16: 80 -16%, 96 -3.5%, 144 -9%, 160 -3%;
// bfloat16: 80 -7%, 96 -2%, 144 and 160 -37% (its padded 32-lane rows held
// only two tokens a wave).  Head_dim 48 (4 passes either way) took 4%
// longer and keeps RowGeo's rows.  Groups of 32 only (the other group sizes
// are head_dim 128).
template <int D> struct KeyRowGeo {
    static constexpr int kChunks = D / 8;
    static constexpr int kPackedRows = 64 / kChunks;
    static constexpr bool kPack = (kChunks & (kChunks - 1)) != 0 &&
                                  (32 + kPackedRows - 1) / kPackedRows < 32 / RowGeo<D>::kRowsPerWave;
    static constexpr int kLanesPerRow = kPack ? kChunks : RowGeo<D>::kLanesPerRow;
    static constexpr int kRowsPerWave = 64 / kLanesPerRow;
};

// One tile.  xt, ct, rt point at token s0 of the slab (input, codes, recon);
// n_rows = min(32, S - s0) real rows.  RAGGED tiles clamp loads to the last
// real row and guard stores; full tiles do neither.
template <int BITS, bool RECON, bool RAGGED, bool BF16, int G, int D, typename MT>
__device__ __forceinline__ void key_tile(const uint16_t* __restrict__ xt, uint32_t* __restrict__ ct,
                                         MT* __restrict__ sct, MT* __restrict__ zet,
                                         uint16_t* __restrict__ rt, int n_rows, int lane, float one,
                                         uint4* __restrict__ xl)
{
    constexpr bool MH = sizeof(MT) == 2;            // binary16 scale/zero
    constexpr int kWords = D * BITS / 32;          // code words per token row
    constexpr bool kPack = KeyRowGeo<D>::kPack;
    static_assert(G == 32 || !kPack, "packed key rows hold groups of 32 only");
    constexpr int kLPR = KeyRowGeo<D>::kLanesPerRow;
    constexpr int kRPW = KeyRowGeo<D>::kRowsPerWave;
    constexpr int kChunks = RowGeo<D>::kChunks;
    const int c = lane % kLPR;                     // channels 8c .. 8c+7
    // lanes past the wave's last whole row (packed rows) take row 0's place
    // and store nothing
    const bool in_row = kLPR * kRPW == 64 || lane < kLPR * kRPW;
    const int r = in_row ? lane / kLPR : 0;        // token rows r, r + kRPW, ...
    // lanes past a row's last chunk (head_dims that are not 64, 128 or 256)
    // re-read that chunk and store nothing; their min/max only meet each
    // other's
    const bool has = (kChunks == kLPR || c < kChunks) && in_row;
    const int cl = kChunks == kLPR ? c : (c < kChunks ? c : kChunks - 1);

    // Load the lane's token rows x 8 channels.  Rows past the end of a ragged last
    // group re-read the last real token, which is the edge padding of
    // "Three ways to be off by one bit", item 3, and cannot move min or max.
    constexpr int kRows = (G + kRPW - 1) / kRPW;   // token rows per lane: the tile is one group
    uint4 raw[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        int row = r + kRPW * i;
        if constexpr (G % kRPW != 0) row = row < G ? row : G - 1;   // a last pass past the group
        if constexpr (RAGGED) row = row < n_rows ? row : n_rows - 1;
        raw[i] = load_stream(xt + row * D + cl * 8);
    }

    // Per-channel min/max over the lane's rows and then across the 4 row
    // lanes: fp16 in packed fp16 (exact: the conversion to fp32 is
    // monotone), bfloat16 widened exactly to fp32 (no packed bfloat16 form).
    float mnf[8], mxf[8];
    if constexpr (!BF16) {
        half2_t mnw[4], mxw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            half2_t mn = as_h2(word_of(raw[0], k)), mx = mn;
#pragma unroll
            for (int i = 1; i < kRows; i += 2) {
                const half2_t a = as_h2(word_of(raw[i], k));
                if (i + 1 < kRows) {
                    const half2_t b = as_h2(word_of(raw[i + 1], k));
                    mn = hmin3(mn, a, b);
                    mx = hmax3(mx, a, b);
                } else {
                    mn = hmin(mn, a);
                    mx = hmax(mx, a);
                }
            }
            if constexpr (!kPack) {
                mn = cross_rows_min<D>(mn);
                mx = cross_rows_max<D>(mx);
                mnf[2 * k] = static_cast<float>(mn[0]); mnf[2 * k + 1] = static_cast<float>(mn[1]);
                mxf[2 * k] = static_cast<float>(mx[0]); mxf[2 * k + 1] = static_cast<float>(mx[1]);
            }
            mnw[k] = mn;
            mxw[k] = mx;
        }
        if constexpr (kPack) {
            // every lane posts its 8 channels' min and max in its own LDS
            // slots; then each folds in the kRPW rows' slots of its chunk (a
            // wave's LDS instructions run in order; the fences keep the
            // compiler from moving them)
            xl[2 * lane] = make_uint4(as_u32(mnw[0]), as_u32(mnw[1]), as_u32(mnw[2]), as_u32(mnw[3]));
            xl[2 * lane + 1] = make_uint4(as_u32(mxw[0]), as_u32(mxw[1]), as_u32(mxw[2]), as_u32(mxw[3]));
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
            for (int rr = 0; rr < kRPW; ++rr) {
                const uint4 a = xl[2 * (rr * kLPR + c)], b = xl[2 * (rr * kLPR + c) + 1];
                const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    mnw[k] = rr == 0 ? as_h2(av[k]) : hmin(mnw[k], as_h2(av[k]));
                    mxw[k] = rr == 0 ? as_h2(bv[k]) : hmax(mxw[k], as_h2(bv[k]));
                }
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                mnf[2 * k] = static_cast<float>(mnw[k][0]); mnf[2 * k + 1] = static_cast<float>(mnw[k][1]);
                mxf[2 * k] = static_cast<float>(mxw[k][0]); mxf[2 * k + 1] = static_cast<float>(mxw[k][1]);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const auto val = [&](int i) {
                const uint32_t w = word_of(raw[i], j >> 1);
                return (j & 1) ? bf16_hi(w) : bf16_lo(w);
            };
            float mn = val(0), mx = mn;
#pragma unroll
            for (int i = 1; i < kRows; i += 2) {
                const float a = val(i);
                if (i + 1 < kRows) {
                    const float b = val(i + 1);
                    mn = fmin3(mn, a, b);
                    mx = fmax3(mx, a, b);
                } else {
                    mn = fminimum(mn, a);
                    mx = fmaximum(mx, a);
                }
            }
            if constexpr (!kPack) {
                mn = cross_rows_min_f32<D>(mn);
                mx = cross_rows_max_f32<D>(mx);
            }
            mnf[j] = mn;
            mxf[j] = mx;
        }
        if constexpr (kPack) {
            // as for fp16: the min and max of bfloat16 elements are bfloat16
            // values, so they travel as bfloat16 pairs, 2 slots a lane
            const auto pair = [](float lo, float hi) {
                return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
            };
            xl[2 * lane] = make_uint4(pair(mnf[0], mnf[1]), pair(mnf[2], mnf[3]), pair(mnf[4], mnf[5]), pair(mnf[6], mnf[7]));
            xl[2 * lane + 1] = make_uint4(pair(mxf[0], mxf[1]), pair(mxf[2], mxf[3]), pair(mxf[4], mxf[5]), pair(mxf[6], mxf[7]));
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
            for (int rr = 0; rr < kRPW; ++rr) {
                const uint4 a = xl[2 * (rr * kLPR + c)], b = xl[2 * (rr * kLPR + c) + 1];
                const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float va = (j & 1) ? bf16_hi(av[j >> 1]) : bf16_lo(av[j >> 1]);
                    const float vb = (j & 1) ? bf16_hi(bv[j >> 1]) : bf16_lo(bv[j >> 1]);
                    mnf[j] = rr == 0 ? va : fminimum(mnf[j], va);
                    mxf[j] = rr == 0 ? vb : fmaximum(mxf[j], vb);
                }
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
    }

    // zero = min, scale = RN((max - min) / (2^bits - 1)), r ~ 1/scale.  (The
    // range needs no zero canonicalization: x - y is +0 for equal zeros.)
    float ze[8], sc[8], rc[8];
    bool slow = false;                              // a scale off the fast path (bfloat16, binary16 metadata)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ze[j] = canon_zero(mnf[j]);
        sc[j] = BF16 ? scale_wide<BITS>(mxf[j] - mnf[j]) : scale_of<BITS>(mxf[j] - mnf[j]);
        if constexpr (MH) {
            sc[j] = round_to_f16(sc[j]);
            slow |= slow_scale16(sc[j], mxf[j] - mnf[j]);
        }
        rc[j] = recip_clamped(sc[j]);
        if constexpr (BF16) slow |= !fast_scale(sc[j]);
    }

    if constexpr (MH) {
        uint32_t h[8];
        if (r == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = f32_to_f16(sc[j]);
            store_stream(sct + c * 8, pack8(h));
        } else if (r == 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = f32_to_f16(ze[j]);
            store_stream(zet + c * 8, pack8(h));
        }
    } else if (has) {
        if (r == 0) {
            store_stream4(sct + c * 8, sc[0], sc[1], sc[2], sc[3]);
            store_stream4(sct + c * 8 + 4, sc[4], sc[5], sc[6], sc[7]);
        } else if (r == 1) {
            store_stream4(zet + c * 8, ze[0], ze[1], ze[2], ze[3]);
            store_stream4(zet + c * 8 + 4, ze[4], ze[5], ze[6], ze[7]);
        }
    }

#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int row = r + kRPW * i;
        float t[8], qf[8];
        if constexpr (BF16) {
            // bfloat16: each element whose quotient lies within 2^-16 of a tie
            // is recomputed with the IEEE quotient (the proof at quant_fast is
            // per element).  A wave runs such a branch only when one of its
            // lanes needs it; bfloat16's coarser grid makes ties about 8 times
            // likelier than fp16's (2e-3 of the elements of the synthetic
            // cache), so a whole-row recompute ran in 65% of a wave's rows.
            float dv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                t[j] = sub_elem<BF16>(raw[i], j, one, ze[j]);
                dv[j] = 0.0f;
                qf[j] = quant_fast(t[j], rc[j], dv[j]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (dv[j] > kNearTie || slow) qf[j] = quant_exact(t[j], sc[j], static_cast<float>((1 << BITS) - 1));
        } else {
            float dev = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                t[j] = sub_elem<BF16>(raw[i], j, one, ze[j]);
                qf[j] = quant_fast(t[j], rc[j], dev);
            }
            if (dev > kNearTie || slow) {          // rare: within 2^-16 of a tie
#pragma unroll
                for (int j = 0; j < 8; ++j) qf[j] = quant_exact(t[j], sc[j], static_cast<float>((1 << BITS) - 1));
            }
        }
        uint32_t packed = static_cast<uint32_t>(qf[0]);
#pragma unroll
        for (int j = 1; j < 8; ++j) packed |= static_cast<uint32_t>(qf[j]) << (BITS * j);
        const bool live = (!RAGGED || row < n_rows) && has && (G % kRPW == 0 || row < G);
        if constexpr (BITS == 4) {
            // the lane's 8 channels are exactly one word
            if (live) store_stream(&ct[row * kWords + c], packed);
        } else {
            // 16 channels per word: the even lane takes its odd neighbour's half
            const uint32_t hi = quad_xor1(packed);
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

template <int BITS, bool RECON, bool BF16, int G, int D, typename MT>
__device__ __forceinline__ void key_flush_body(
    const uint16_t* __restrict__ x, int64_t S, int64_t x_bh_stride,
    uint32_t* __restrict__ codes, int64_t codes_bh_stride,
    MT* __restrict__ scale, MT* __restrict__ zero, int64_t meta_bh_stride,
    int64_t dst_token, uint16_t* __restrict__ recon, int64_t recon_bh_stride,
    int64_t n_groups, int64_t n_tiles, float one)
{
    constexpr int kWords = D * BITS / 32;
    const int lane = threadIdx.x & 63;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;                   // uniform across the wave
    const int64_t bh = tile / n_groups;
    const int64_t g = tile - bh * n_groups;
    const int64_t s0 = g * G;
    const uint16_t* xt = x + bh * x_bh_stride + s0 * D;
    uint32_t* ct = codes + bh * codes_bh_stride + (dst_token + s0) * kWords;
    const int64_t moff = bh * meta_bh_stride + (dst_token / G + g) * D;
    uint16_t* rt = RECON ? recon + bh * recon_bh_stride + s0 * D : nullptr;
    const int64_t rows = S - s0;
    uint4* xl = nullptr;
    if constexpr (KeyRowGeo<D>::kPack) {
        // the wave's min/max exchange of packed rows (static LDS only where
        // rows are packed, so the capped head_dim-128 launches keep theirs)
        __shared__ uint4 key_xchg[kWavesPerBlock][128];   // a lane's min and max: 2 slots
        xl = key_xchg[threadIdx.x >> 6];
    }
    if (rows >= G)
        key_tile<BITS, RECON, false, BF16, G, D, MT>(xt, ct, scale + moff, zero + moff, rt, G, lane, one, xl);
    else
        key_tile<BITS, RECON, true, BF16, G, D, MT>(xt, ct, scale + moff, zero + moff, rt, static_cast<int>(rows), lane, one, xl);
}

template <int BITS, bool RECON, bool BF16, int G, int D, typename MT>
__global__ __launch_bounds__(kBlock) void key_flush_kernel(
    const uint16_t* __restrict__ x, int64_t S, int64_t x_bh_stride,
    uint32_t* __restrict__ codes, int64_t codes_bh_stride,
    MT* __restrict__ scale, MT* __restrict__ zero, int64_t meta_bh_stride,
    int64_t dst_token, uint16_t* __restrict__ recon, int64_t recon_bh_stride,
    int64_t n_groups, int64_t n_tiles, float one)
{
    key_flush_body<BITS, RECON, BF16, G, D, MT>(x, S, x_bh_stride, codes, codes_bh_stride, scale, zero, meta_bh_stride, dst_token, recon, recon_bh_stride, n_groups, n_tiles, one);
}

// bfloat16 keys with more than 8 token rows per lane held about 200
// registers (2 waves per SIMD) at head_dims above 160 and about 150 (3) in
// the packed rows of 144 and 160.  This entry caps the registers: 3 waves
// for the 32-lane rows (a few spills), 4 for the packed rows.  Interleaved
// A/B on MI355X, 4-bit bfloat16 keys, 32768 tokens per slab: 176, 192 and
// 224 -23 to -25%, 256 -16%, 144 -13%, 160 -9%; a cap of 4 on the 32-lane
// rows spilled 330-400 bytes a lane and doubled their time.
template <int D> constexpr int kKeyWavesBF16 =
    (32 + KeyRowGeo<D>::kRowsPerWave - 1) / KeyRowGeo<D>::kRowsPerWave <= 8 ? 0 : KeyRowGeo<D>::kPack ? 4 : 3;
template <int BITS, bool RECON, bool BF16, int G, int D, typename MT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kKeyWavesBF16<D>)))
void key_flush_capped_kernel(
    const uint16_t* __restrict__ x, int64_t S, int64_t x_bh_stride,
    uint32_t* __restrict__ codes, int64_t codes_bh_stride,
    MT* __restrict__ scale, MT* __restrict__ zero, int64_t meta_bh_stride,
    int64_t dst_token, uint16_t* __restrict__ recon, int64_t recon_bh_stride,
    int64_t n_groups, int64_t n_tiles, float one)
{
    key_flush_body<BITS, RECON, BF16, G, D, MT>(x, S, x_bh_stride, codes, codes_bh_stride, scale, zero, meta_bh_stride, dst_token, recon, recon_bh_stride, n_groups, n_tiles, one);
}

// ---------------------------------------------------------------------------
// Values: group = (bh, token s, channel group j) over channels [32j, 32j+32)
// ---------------------------------------------------------------------------

// Whether a value tile gathers its tokens' scale and zero in LDS and writes
// them as one store per array (a token per lane) instead of the plain
// per-group stores of the reduction lanes.  Measured on the full 32k cache:
// with 16 or 32 bytes per token (groups of 32, binary32) the gathered,
// nontemporal stores made the 4-bit value flush 7% faster (0.599 -> 0.559
// ms) and the 2-bit one 5%; with 4 to 8 bytes per token (groups of 64 or
// 128, or binary16 scale/zero) they made it 8-10% slower, and those keep
// the plain stores, whose partial lines the L2 merges.
// Value groups per token: a head_dim that G does not divide ends each token
// with a shorter group.
template <int G, int D> constexpr int kGroupsPerTok = (D + G - 1) / G;
// Gathered: 16 to 32 bytes of scale (and of zero) per token.  The rows of
// 20, 24 and 28 bytes (head_dims 144 to 224) leave as dword stores of
// consecutive lanes, which ran those value flushes 3-5% faster than plain
// stores; at 12 bytes (head_dims 80 and 96) gathering was 1-3% slower.
template <int G, int D, typename MT>
constexpr bool kGatherMeta = kGroupsPerTok<G, D> * static_cast<int>(sizeof(MT)) >= 16 &&
                             kGroupsPerTok<G, D> * static_cast<int>(sizeof(MT)) <= 32;
// Elements of a wave's LDS row for the gathered scale and zero (one element
// when nothing is gathered), and the workgroup's static LDS bytes.
template <int G, int D, typename MT>
constexpr int kValueLdsRow = kGatherMeta<G, D, MT> ? 2 * 32 * kGroupsPerTok<G, D> : 1;
template <int G, int D, typename MT>
constexpr size_t kValueLdsBytes = sizeof(MT) * kWavesPerBlock * kValueLdsRow<G, D, MT>;

// One token's scale (or zero) row, 16 or 32 bytes, from LDS to the store
// (16-byte aligned: the store's metadata is, and so is a token's row).
template <int BYTES>
__device__ __forceinline__ void meta_row_out(const void* src, void* dst) {
    static_assert(BYTES == 16 || BYTES == 32, "gathered rows are 16 or 32 bytes");
    const uint4* s = static_cast<const uint4*>(src);
    u32x4_t* d = static_cast<u32x4_t*>(dst);
#pragma unroll
    for (int k = 0; k < BYTES / 16; ++k) {
        const uint4 a = s[k];
        __builtin_nontemporal_store(u32x4_t{a.x, a.y, a.z, a.w}, d + k);
    }
}
// With kGatherMeta, the tile's 32 tokens of scale and zero are gathered in
// the wave's LDS rows (lds: 2 x 32 x D/G elements) and leave in one store
// per array, a token per lane: 32 x D/G x sizeof(MT) contiguous bytes, whole
// lines.
// Value rows.  A value group of 32 channels is one DPP quad and no exchange
// crosses token rows, so a row needs whole quads, not a power-of-two lane
// count: head_dims 80 and 96 can take rows of 12 lanes (5 tokens a wave
// instead of 4), 144 and 160 rows of 20 (3 instead of 2).  Measured against
// RowGeo's rows: 144 19-20% and 160 14% faster; 80 12% faster over 256
// slabs of 32768 tokens and level over 460; 96 11% faster for bfloat16
// caches but 5% slower for fp16 ones, which keep RowGeo's 16-lane rows; the
// other head_dims gain no rows.
template <int D, bool BF16> struct ValueRowGeo {
    static constexpr int kChunks = D / 8;
    static constexpr int kQuadLanes = (kChunks + 3) / 4 * 4;
    static constexpr bool kPack = 64 / kQuadLanes > RowGeo<D>::kRowsPerWave && (BF16 || D != 96);
    static constexpr int kLanesPerRow = kPack ? kQuadLanes : RowGeo<D>::kLanesPerRow;
    static constexpr int kRowsPerWave = 64 / kLanesPerRow;
};

template <int BITS, bool RECON, bool RAGGED, bool BF16, int G, int D, typename MT>
__device__ __forceinline__ void value_tile(const uint16_t* __restrict__ xt, uint32_t* __restrict__ ct,
                                           MT* __restrict__ sct, MT* __restrict__ zet,
                                           uint16_t* __restrict__ rt, int n_rows, int lane, float one,
                                           MT* __restrict__ lds)
{
    constexpr bool MH = sizeof(MT) == 2;            // binary16 scale/zero
    constexpr int kWords = D * BITS / 32;
    constexpr int kMetaPerTok = kGroupsPerTok<G, D>;   // channel groups per token
    constexpr int kLanesPerGroup = G / 8;           // 4, 8 or 16 lanes of 8 channels
    constexpr int kLPR = ValueRowGeo<D, BF16>::kLanesPerRow;
    constexpr int kRPW = ValueRowGeo<D, BF16>::kRowsPerWave;
    constexpr int kChunks = ValueRowGeo<D, BF16>::kChunks;
    constexpr int kRows = (32 + kRPW - 1) / kRPW;   // token rows per lane in a 32-token tile
    static_assert(G == 32 || !ValueRowGeo<D, BF16>::kPack, "rows of whole quads hold groups of 32 only");
    const int c = lane % kLPR;
    // lanes past the wave's last whole row (rows of 12 or 20 lanes) take row
    // 0's place in every pass and store nothing
    const bool in_row = kLPR * kRPW == 64 || lane < kLPR * kRPW;
    const int r = in_row ? lane / kLPR : 0;
    const int j = c / kLanesPerGroup;               // channel group of this lane
    // lanes past a row's last chunk (head_dims that are not 64, 128 or 256)
    // re-read that chunk and store nothing: in a quad they share with a
    // ragged last group (16 channels) they repeat its last chunk, which
    // cannot move the group's min or max
    const bool has = kChunks == kLPR || c < kChunks;
    const int cl = kChunks == kLPR ? c : (c < kChunks ? c : kChunks - 1);

    uint4 raw[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        int row = r + kRPW * i;
        if (32 % kRPW != 0) row = row < 32 ? row : 31;                  // a last pass past the tile
        if constexpr (RAGGED) row = row < n_rows ? row : n_rows - 1;   // keep every lane in the exchange
        raw[i] = load_stream(xt + row * D + cl * 8);
    }

#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int row = r + kRPW * i;
        const bool in_tile = in_row && (32 % kRPW == 0 || row < 32);   // a real token row of the tile
        float lo, hi;
        if constexpr (!BF16) {
            const half2_t hv[4] = {as_h2(raw[i].x), as_h2(raw[i].y), as_h2(raw[i].z), as_h2(raw[i].w)};
            const half2_t mn2 = hmin(hmin3(hv[0], hv[1], hv[2]), hv[3]);
            const half2_t mx2 = hmax(hmax3(hv[0], hv[1], hv[2]), hv[3]);
            // (min, -max) of the lane in one register, then the 4 lanes of the
            // group (a DPP quad) with min only
            half2_t mm;
            mm[0] = __builtin_elementwise_minimum(mn2[0], mn2[1]);
            mm[1] = -__builtin_elementwise_maximum(mx2[0], mx2[1]);
            mm = hmin(mm, as_h2(quad_xor1(as_u32(mm))));
            mm = hmin(mm, as_h2(quad_xor2(as_u32(mm))));
            if constexpr (G >= 64) mm = hmin(mm, as_h2(half_row_mirror(as_u32(mm))));
            if constexpr (G >= 128) mm = hmin(mm, as_h2(row_mirror(as_u32(mm))));
            lo = static_cast<float>(mm[0]);
            hi = -static_cast<float>(mm[1]);
        } else {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t w = word_of(raw[i], k >> 1);
                v[k] = (k & 1) ? bf16_hi(w) : bf16_lo(w);
            }
            lo = fminimum(fmin3(v[0], v[1], v[2]), fmin3(v[3], v[4], v[5]));
            lo = fmin3(lo, v[6], v[7]);
            hi = fmaximum(fmax3(v[0], v[1], v[2]), fmax3(v[3], v[4], v[5]));
            hi = fmax3(hi, v[6], v[7]);
            lo = fminimum(lo, __uint_as_float(quad_xor1(__float_as_uint(lo))));
            hi = fmaximum(hi, __uint_as_float(quad_xor1(__float_as_uint(hi))));
            lo = fminimum(lo, __uint_as_float(quad_xor2(__float_as_uint(lo))));
            hi = fmaximum(hi, __uint_as_float(quad_xor2(__float_as_uint(hi))));
            if constexpr (G >= 64) {
                lo = fminimum(lo, __uint_as_float(half_row_mirror(__float_as_uint(lo))));
                hi = fmaximum(hi, __uint_as_float(half_row_mirror(__float_as_uint(hi))));
            }
            if constexpr (G >= 128) {
                lo = fminimum(lo, __uint_as_float(row_mirror(__float_as_uint(lo))));
                hi = fmaximum(hi, __uint_as_float(row_mirror(__float_as_uint(hi))));
            }
        }
        const float ze = canon_zero(lo);
        float sc = BF16 ? scale_wide<BITS>(hi - lo) : scale_of<BITS>(hi - lo);
        if constexpr (MH) sc = round_to_f16(sc);
        const float rc = recip_clamped(sc);

        float t[8], qf[8];
        if constexpr (BF16) {
            // per element, as in key_tile
            const bool slow = !fast_scale(sc);
            float dv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                t[k] = sub_elem<BF16>(raw[i], k, one, ze);
                dv[k] = 0.0f;
                qf[k] = quant_fast(t[k], rc, dv[k]);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (dv[k] > kNearTie || slow) qf[k] = quant_exact(t[k], sc, static_cast<float>((1 << BITS) - 1));
        } else {
            float dev = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                t[k] = sub_elem<BF16>(raw[i], k, one, ze);
                qf[k] = quant_fast(t[k], rc, dev);
            }
            if (dev > kNearTie || (MH && slow_scale16(sc, hi - lo))) {
#pragma unroll
                for (int k = 0; k < 8; ++k) qf[k] = quant_exact(t[k], sc, static_cast<float>((1 << BITS) - 1));
            }
        }
        uint32_t packed = static_cast<uint32_t>(qf[0]);
#pragma unroll
        for (int k = 1; k < 8; ++k) packed |= static_cast<uint32_t>(qf[k]) << (BITS * k);
        const bool live = (!RAGGED || row < n_rows) && has && in_tile;
        if constexpr (BITS == 4) {
            if (live) store_stream(&ct[row * kWords + c], packed);
        } else {
            const uint32_t hw = quad_xor1(packed);
            if (live && (c & 1) == 0) store_stream(&ct[row * kWords + (c >> 1)], packed | (hw << 16));
        }
        if constexpr (kGatherMeta<G, D, MT>) {
            // to the wave's LDS rows (rows past a ragged end are never copied out)
            if (has && in_tile && c % kLanesPerGroup == 0) lds[row * kMetaPerTok + j] = sc;
            else if (has && in_tile && c % kLanesPerGroup == 1) lds[(32 + row) * kMetaPerTok + j] = ze;
        } else if (live) {
            // plain stores: one instruction writes 16-64 B of a line, which the
            // L2 merges (with the nontemporal hint they reached HBM as partial
            // lines: 8% more write traffic and a slower flush)
            if constexpr (MH) {
                if (c % kLanesPerGroup == 0) sct[row * kMetaPerTok + j] = static_cast<uint16_t>(f32_to_f16(sc));
                else if (c % kLanesPerGroup == 1) zet[row * kMetaPerTok + j] = static_cast<uint16_t>(f32_to_f16(ze));
            } else {
                if (c % kLanesPerGroup == 0) sct[row * kMetaPerTok + j] = sc;
                else if (c % kLanesPerGroup == 1) zet[row * kMetaPerTok + j] = ze;
            }
        }
        if constexpr (RECON) {
            uint32_t h[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) h[k] = recon_out<BF16>(qf[k], sc, ze);
            if (live) store_stream(rt + row * D + c * 8, pack8(h));
        }
    }
    if constexpr (kGatherMeta<G, D, MT>) {
        // one wave: its LDS writes above complete before these reads (a
        // wave's LDS instructions run in order; the fence keeps the compiler
        // from moving them)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        constexpr int kBytes = kMetaPerTok * static_cast<int>(sizeof(MT));
        if constexpr (kBytes == 16 || kBytes == 32) {
            if (lane < 32 && (!RAGGED || lane < n_rows)) {
                meta_row_out<kBytes>(lds + lane * kMetaPerTok, sct + lane * kMetaPerTok);
                meta_row_out<kBytes>(lds + (32 + lane) * kMetaPerTok, zet + lane * kMetaPerTok);
            }
        } else {
            // 20 to 28 bytes per token (rows not 16-byte aligned): the words
            // leave in order, one per lane, so consecutive lanes fill whole
            // lines
            static_assert(sizeof(MT) == 4, "gathered binary16 rows are 16 or 32 bytes");
            const int n_words = (RAGGED ? n_rows : 32) * kMetaPerTok;
#pragma unroll
            for (int it = 0; it < (32 * kMetaPerTok + 63) / 64; ++it) {
                const int w = lane + 64 * it;
                if (w < n_words) {
                    store_stream(&sct[w], lds[w]);
                    store_stream(&zet[w], lds[32 * kMetaPerTok + w]);
                }
            }
        }
    }
}

template <int BITS, bool RECON, bool BF16, int G, int D, typename MT>
__global__ __launch_bounds__(kBlock) void value_flush_kernel(
    const uint16_t* __restrict__ x, int64_t S, int64_t x_bh_stride,
    uint32_t* __restrict__ codes, int64_t codes_bh_stride,
    MT* __restrict__ scale, MT* __restrict__ zero, int64_t meta_bh_stride,
    int64_t dst_token, uint16_t* __restrict__ recon, int64_t recon_bh_stride,
    int64_t tiles_per_bh, int64_t n_tiles, float one)
{
    constexpr int kWords = D * BITS / 32;
    constexpr int kMetaPerTok = kGroupsPerTok<G, D>;
    const int lane = threadIdx.x & 63;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    __shared__ MT lds_meta[kWavesPerBlock][kValueLdsRow<G, D, MT>];
    static_assert(sizeof(lds_meta) == kValueLdsBytes<G, D, MT>, "the launcher sizes its LDS cap from this");
    if (tile >= n_tiles) return;                    // uniform across the wave
    const int64_t bh = tile / tiles_per_bh;
    const int64_t s0 = (tile - bh * tiles_per_bh) * 32;
    const uint16_t* xt = x + bh * x_bh_stride + s0 * D;
    uint32_t* ct = codes + bh * codes_bh_stride + (dst_token + s0) * kWords;
    const int64_t moff = bh * meta_bh_stride + (dst_token + s0) * kMetaPerTok;
    uint16_t* rt = RECON ? recon + bh * recon_bh_stride + s0 * D : nullptr;
    const int64_t rows = S - s0;
    MT* lds = lds_meta[threadIdx.x >> 6];
    if (rows >= 32)
        value_tile<BITS, RECON, false, BF16, G, D, MT>(xt, ct, scale + moff, zero + moff, rt, 32, lane, one, lds);
    else
        value_tile<BITS, RECON, true, BF16, G, D, MT>(xt, ct, scale + moff, zero + moff, rt, static_cast<int>(rows), lane, one, lds);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

// Workgroups a flush lets reside on one CU (0: as many as its registers
// allow, 8 for these kernels).  A cap is held by LDS the launch reserves and
// never touches (160 KiB per CU on gfx950).  Measured on the full 32k cache,
// interleaved against the uncapped kernels: at fp16 input and head_dim 128
// the key flush ran 2-3% faster at 5 per CU (4 bits, groups of 32; 5% at 2
// bits, 7% with binary16 scale/zero) and the value flush whose scale and
// zero go out through LDS (groups of 32, binary32) 5-6% faster at 4 per CU,
// as the streaming calibration kernels did; fewer requests in flight at once
// suit the memory system.  bfloat16 input, head_dim 64 and the
// reconstructing flushes ran 1-7% slower with a cap, and the other value
// configurations 2-5% slower, so they keep the full residency.
// At head_dim 256 (16 KiB of input per wave) 3 per CU ran the key flush 3%
// and the value flush 2% faster than the 4 its registers allow; the head_dims
// with idle lanes at the end of each row ran 5-90% slower with a cap of 3
// or 4 and keep the full residency.
template <bool KEYS, bool RECON, bool BF16, int G, int D, typename MT>
constexpr int kFlushPerCU = (BF16 || RECON) ? 0
                            : D == 256 ? 3
                            : D != 128 ? 0
                            : KEYS ? 5 : (kGatherMeta<G, D, MT> ? 4 : 0);

// The dynamic LDS bytes that hold a launch to per_cu workgroups per CU, on
// top of static_bytes of its own (0 for no cap).
static size_t residency_lds(int per_cu, size_t static_bytes) {
    if (per_cu <= 0) return 0;
    const size_t per_block = (size_t{160} * 1024 / static_cast<size_t>(per_cu)) / 1024 * 1024;
    return per_block > static_bytes ? per_block - static_bytes : 0;
}

template <int BITS, bool RECON, bool BF16, int G, int D, typename MT>
static hipError_t launch_keys_t(const FlushArgs& a, hipStream_t stream) {
    const int64_t n_groups = (a.S + G - 1) / G;
    const int64_t n_tiles = a.BH * n_groups;
    const int64_t blocks = (n_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const size_t lds = residency_lds(kFlushPerCU<true, RECON, BF16, G, D, MT>, 0);
    if constexpr (BF16 && kKeyWavesBF16<D> > 0)
        hipLaunchKernelGGL((key_flush_capped_kernel<BITS, RECON, BF16, G, D, MT>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kBlock), lds, stream, a.x, a.S, a.x_bh_stride, a.codes,
                           a.codes_bh_stride, static_cast<MT*>(a.scale), static_cast<MT*>(a.zero),
                           a.meta_bh_stride, a.dst_token,
                           a.recon, a.recon_bh_stride, n_groups, n_tiles, 1.0f);
    else
        hipLaunchKernelGGL((key_flush_kernel<BITS, RECON, BF16, G, D, MT>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kBlock), lds, stream, a.x, a.S, a.x_bh_stride, a.codes,
                           a.codes_bh_stride, static_cast<MT*>(a.scale), static_cast<MT*>(a.zero),
                           a.meta_bh_stride, a.dst_token,
                           a.recon, a.recon_bh_stride, n_groups, n_tiles, 1.0f);
    return hipGetLastError();
}

template <int BITS, bool RECON, bool BF16, int G, int D, typename MT>
static hipError_t launch_values_t(const FlushArgs& a, hipStream_t stream) {
    const int64_t tiles_per_bh = (a.S + 31) / 32;
    const int64_t n_tiles = a.BH * tiles_per_bh;
    const int64_t blocks = (n_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const size_t lds = residency_lds(kFlushPerCU<false, RECON, BF16, G, D, MT>, kValueLdsBytes<G, D, MT>);
    hipLaunchKernelGGL((value_flush_kernel<BITS, RECON, BF16, G, D, MT>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kBlock), lds, stream, a.x, a.S, a.x_bh_stride, a.codes,
                       a.codes_bh_stride, static_cast<MT*>(a.scale), static_cast<MT*>(a.zero),
                       a.meta_bh_stride, a.dst_token,
                       a.recon, a.recon_bh_stride, tiles_per_bh, n_tiles, 1.0f);
    return hipGetLastError();
}

// One instantiation per (bits, reconstruction, input format, group size,
// head_dim, metadata format).
template <bool KEYS, bool BF16, int G, int D, typename MT = float>
static hipError_t launch_flush_g(const FlushArgs& a, hipStream_t stream) {
    const bool rec = a.recon != nullptr;
    if constexpr (KEYS) {
        if (a.bits == 4) return rec ? launch_keys_t<4, true, BF16, G, D, MT>(a, stream) : launch_keys_t<4, false, BF16, G, D, MT>(a, stream);
        return rec ? launch_keys_t<2, true, BF16, G, D, MT>(a, stream) : launch_keys_t<2, false, BF16, G, D, MT>(a, stream);
    } else {
        if (a.bits == 4) return rec ? launch_values_t<4, true, BF16, G, D, MT>(a, stream) : launch_values_t<4, false, BF16, G, D, MT>(a, stream);
        return rec ? launch_values_t<2, true, BF16, G, D, MT>(a, stream) : launch_values_t<2, false, BF16, G, D, MT>(a, stream);
    }
}

// head_dim 128 with groups of 32, 64 or 128; every other multiple of 16 up
// to 256 with groups of 32 (the ABI admits no other pair).  Binary16
// metadata: fp16 input at head_dim 128.
template <bool KEYS, bool BF16>
static hipError_t launch_flush_fmt(const FlushArgs& a, hipStream_t stream) {
    switch (a.head_dim) {
#define KIVI_FLUSH_D(D) case D: return launch_flush_g<KEYS, BF16, 32, D>(a, stream);
        KIVI_FLUSH_D(16) KIVI_FLUSH_D(32) KIVI_FLUSH_D(48) KIVI_FLUSH_D(64) KIVI_FLUSH_D(80)
        KIVI_FLUSH_D(96) KIVI_FLUSH_D(112) KIVI_FLUSH_D(144) KIVI_FLUSH_D(160) KIVI_FLUSH_D(176)
        KIVI_FLUSH_D(192) KIVI_FLUSH_D(208) KIVI_FLUSH_D(224) KIVI_FLUSH_D(240) KIVI_FLUSH_D(256)
#undef KIVI_FLUSH_D
        default: break;
    }
    if constexpr (!BF16) {
        if (a.meta16) {
            switch (a.group) {
                case 64: return launch_flush_g<KEYS, false, 64, 128, uint16_t>(a, stream);
                case 128: return launch_flush_g<KEYS, false, 128, 128, uint16_t>(a, stream);
                default: return launch_flush_g<KEYS, false, 32, 128, uint16_t>(a, stream);
            }
        }
    }
    switch (a.group) {
        case 64: return launch_flush_g<KEYS, BF16, 64, 128>(a, stream);
        case 128: return launch_flush_g<KEYS, BF16, 128, 128>(a, stream);
        default: return launch_flush_g<KEYS, BF16, 32, 128>(a, stream);
    }
}

// Every head_dim the ABI admits (multiples of 16 up to 256) runs on the tiled
// kernels: rows of 8, 16 or 32 lanes, idle at the end when D/8 is not a
// power of two.  The ABI rejects other head_dims before any launch.
static bool tiled_head_dim(int D) { return D >= 16 && D <= 256 && D % 16 == 0; }

hipError_t launch_key_flush(const FlushArgs& a, hipStream_t stream) {
    if (!tiled_head_dim(a.head_dim)) return hipErrorInvalidValue;
    return a.bf16 ? launch_flush_fmt<true, true>(a, stream) : launch_flush_fmt<true, false>(a, stream);
}

hipError_t launch_value_flush(const FlushArgs& a, hipStream_t stream) {
    if (!tiled_head_dim(a.head_dim)) return hipErrorInvalidValue;
    return a.bf16 ? launch_flush_fmt<false, true>(a, stream) : launch_flush_fmt<false, false>(a, stream);
}

}  // namespace kivi
