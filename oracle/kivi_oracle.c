/*
 * kivi_oracle.c -- plain, slow, single-threaded CPU oracle for the KIVI
 * KV-cache flush (per-channel keys, per-token values), its dequantization,
 * and dequantize-then-attend decode.
 *
 * TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
 * cpu_baseline leg are its only users.  It shares nothing with the HIP
 * library (no source, header, table or generator).
 *
 * Sources, cited by page title and section:
 *   [Metal post]  "A 5.65x Metal Kernel That Made My LLM Exactly 0% Faster"
 *                 (VeloxQuant-MLX blog)
 *   [Qwen3 post]  "A Kernel That Wasn't There" (VeloxQuant-MLX blog)
 *   [Benchmarks]  VeloxQuant-MLX "Benchmarks" page
 *
 * Build flags matter for what this file computes: it must be compiled with
 * -ffp-contract=off (a multiply feeding an add stays two roundings, as
 * [Metal post] "Three ways to be off by one bit", item 1, requires) and
 * without -ffast-math, in the default round-to-nearest-even mode, with SSE
 * float arithmetic (x86-64 default), so every float operation below is one
 * correctly rounded IEEE binary32 operation.
 */
#include "kivi_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must not be built with -ffast-math"
#endif

/* ------------------------------------------------------------------ */
/* IEEE binary16 codec, written from the format's definition:         */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.           */
/* ------------------------------------------------------------------ */

float orc_f16_to_f32(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    float mag;
    if (expo == 0) {
        /* zero or subnormal: frac * 2^-24 (exact in binary32) */
        mag = ldexpf((float)frac, -24);
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        /* normal: (1024 + frac) * 2^(expo - 25) (exact in binary32) */
        mag = ldexpf((float)(1024 + frac), expo - 25);
    }
    return sign ? -mag : mag;
}

/* round a non-negative double holding at most 53 significant bits to the
   nearest integer, ties to even */
static double round_half_even(double n)
{
    const double fl = floor(n);
    const double fr = n - fl;            /* exact */
    if (fr > 0.5) return fl + 1.0;
    if (fr < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t orc_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if ((bits & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(sign | 0x7e00u); /* NaN */
    const double a = fabs((double)f);     /* exact */
    /* 65520 = 65504 + half an ulp: from there on the nearest-even result is
       infinity (the tie at 65520 goes to the even "next" value 2^16) */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; a result of 1024 is the smallest
           normal, whose encoding is the same integer */
        const double r = round_half_even(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)r);
    }
    int k;
    (void)frexp(a, &k);                   /* a = m * 2^k, m in [0.5, 1) */
    const int e = k - 1;                  /* 2^e <= a < 2^(e+1), -14 <= e <= 15 */
    const double r = round_half_even(ldexp(a, 10 - e)); /* in [1024, 2048] */
    /* r == 2048 carries into the exponent field, which this sum does */
    const uint32_t enc = ((uint32_t)(e + 15) << 10) + ((uint32_t)r - 1024u);
    return (uint16_t)(sign | enc);
}

/* ------------------------------------------------------------------ */
/* bfloat16 codec, written from the format's definition: 1 sign bit,  */
/* 8 exponent bits (bias 127), 7 fraction bits -- binary32 with the   */
/* low 16 fraction bits dropped.                                      */
/* ------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t b)
{
    const int sign = (b >> 15) & 1;
    const int expo = (b >> 7) & 0xff;
    const int frac = b & 0x7f;
    float mag;
    if (expo == 0) {
        /* zero or subnormal: frac * 2^-133 (exact in binary32) */
        mag = ldexpf((float)frac, -133);
    } else if (expo == 255) {
        mag = frac ? NAN : INFINITY;
    } else {
        /* normal: (128 + frac) * 2^(expo - 134) (exact in binary32) */
        mag = ldexpf((float)(128 + frac), expo - 134);
    }
    return sign ? -mag : mag;
}

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if ((bits & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(sign | 0x7fc0u); /* NaN */
    if ((bits & 0x7fffffffu) == 0x7f800000u) return (uint16_t)(sign | 0x7f80u);
    const double a = fabs((double)f);     /* exact */
    /* from (2 - 2^-8) * 2^127, half an ulp above the largest finite bfloat16,
       the nearest-even result is infinity (the tie goes to the even 2^128) */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7f80u);
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: quantum 2^-133; a result of 128 is the smallest
           normal, whose encoding is the same integer */
        const double r = round_half_even(ldexp(a, 133));
        return (uint16_t)(sign | (uint16_t)r);
    }
    int k;
    (void)frexp(a, &k);                   /* a = m * 2^k, m in [0.5, 1) */
    const int e = k - 1;                  /* 2^e <= a < 2^(e+1), -126 <= e <= 127 */
    const double r = round_half_even(ldexp(a, 7 - e));  /* in [128, 256] */
    /* r == 256 carries into the exponent field, which this sum does */
    const uint32_t enc = ((uint32_t)(e + 127) << 7) + ((uint32_t)r - 128u);
    return (uint16_t)(sign | enc);
}

void orc_bf16_to_f32_array(const uint16_t *h, float *f, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) f[i] = orc_bf16_to_f32(h[i]);
}

void orc_f32_to_bf16_array(const float *f, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) h[i] = orc_f32_to_bf16(f[i]);
}

/* the 16-bit storage format of inputs and reconstructions */
typedef float (*widen_fn)(uint16_t);
typedef uint16_t (*narrow_fn)(float);
static widen_fn widen_of(int fmt) { return fmt == ORC_BF16 ? orc_bf16_to_f32 : orc_f16_to_f32; }
static narrow_fn narrow_of(int fmt) { return fmt == ORC_BF16 ? orc_f32_to_bf16 : orc_f32_to_f16; }

void orc_f16_to_f32_array(const uint16_t *h, float *f, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) f[i] = orc_f16_to_f32(h[i]);
}

void orc_f32_to_f16_array(const float *f, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) h[i] = orc_f32_to_f16(f[i]);
}

/* ------------------------------------------------------------------ */
/* One group: asymmetric min/max quantization.                        */
/* [Metal post], "What we're actually optimizing": zero is the group  */
/* minimum, scale is (max - min) / (2^bits - 1), the code is the      */
/* rounded (x - zero) / scale, the reconstruction is code*scale+zero; */
/* the reference path runs min, max, subtract, divide, round, clip,   */
/* multiply, add, in that order, each as its own fp32 operation.      */
/* ------------------------------------------------------------------ */

void orc_quantize_group_meta(const uint16_t *x, int n, int bits, int fmt, int meta,
                             float *scale_out, float *zero_out, uint8_t *q, uint16_t *recon)
{
    const widen_fn widen = widen_of(fmt);
    /* widen exactly to fp32 (the Metal kernels read float(x[...]),
       [Metal post] "Kernel A" and "Kernel B") */
    float mn = widen(x[0]);
    float mx = mn;
    for (int i = 1; i < n; ++i) {
        const float v = widen(x[i]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    /* A zero extreme is stored as +0 so the result does not depend on which
       of -0 / +0 a reduction happened to keep (the pages are silent). */
    if (mn == 0.0f) mn = 0.0f;
    if (mx == 0.0f) mx = 0.0f;

    const float levels = (float)((1 << bits) - 1);
    const float range = mx - mn;
    float scale = range / levels;
    float zero = mn;
    if (meta == ORC_META_F16) {
        /* Binary16 metadata: the pair is stored rounded to nearest even
           binary16, and the codes and the reconstruction use the stored
           values, so that a reader of the store reproduces them.  (The zero
           of an fp16 group is an fp16 value already; a scale below 2^-25
           becomes 0 and the group codes as constant.) */
        scale = orc_f16_to_f32(orc_f32_to_f16(scale));
        zero = orc_f16_to_f32(orc_f32_to_f16(zero));
    }
    *scale_out = scale;
    *zero_out = zero;

    for (int i = 0; i < n; ++i) {
        const float v = widen(x[i]);
        int code;
        if (scale == 0.0f) {
            /* constant group: the quotient would be 0/0; every element
               equals zero, so code 0 reconstructs it exactly */
            code = 0;
        } else {
            const float t = v - zero;             /* subtract */
            const float u = t / scale;            /* divide (IEEE) */
            float r = rintf(u);                   /* round: ties to even,
                                                     [Metal post] "Three ways to
                                                     be off by one bit", item 2 */
            if (r < 0.0f) r = 0.0f;               /* clip to [0, 2^bits - 1] */
            if (r > levels) r = levels;
            code = (int)r;
        }
        q[i] = (uint8_t)code;
        if (recon) recon[i] = orc_dequantize_one_fmt((uint32_t)code, scale, zero, fmt);
    }
}

void orc_quantize_group_fmt(const uint16_t *x, int n, int bits, int fmt,
                            float *scale_out, float *zero_out, uint8_t *q, uint16_t *recon)
{
    orc_quantize_group_meta(x, n, bits, fmt, ORC_META_F32, scale_out, zero_out, q, recon);
}

void orc_quantize_group(const uint16_t *x, int n, int bits,
                        float *scale_out, float *zero_out, uint8_t *q, uint16_t *recon)
{
    orc_quantize_group_fmt(x, n, bits, ORC_F16, scale_out, zero_out, q, recon);
}

/* [Metal post], "Three ways to be off by one bit", item 1: the product is
   rounded before the add (no fused multiply-add); the cast to the 16-bit
   format rounds to nearest even. */
uint16_t orc_dequantize_one_fmt(uint32_t q, float scale, float zero, int fmt)
{
    const float prod = (float)q * scale;
    const float sum = prod + zero;
    return narrow_of(fmt)(sum);
}

uint16_t orc_dequantize_one(uint32_t q, float scale, float zero)
{
    return orc_dequantize_one_fmt(q, scale, zero, ORC_F16);
}

/* ------------------------------------------------------------------ */
/* Tensor-level flushes over [BH][S][D] (the flattened [B,H,S,D] cache, */
/* [Metal post] "The layout problem that shapes everything").         */
/* ------------------------------------------------------------------ */

static int check_common(int64_t BH, int64_t S, int64_t D, int bits, int G)
{
    if (BH < 0 || S < 0 || D <= 0 || G <= 0) return -1;
    if (bits != 2 && bits != 4 && bits != 8) return -1;
    if (D % (32 / bits) != 0) return -1;
    return 0;
}

static void put_code(uint32_t *row_words, int64_t d, int bits, uint32_t code)
{
    const int64_t per_word = 32 / bits;
    const int shift = (int)(d % per_word) * bits;
    row_words[d / per_word] |= code << shift;
}

/* Keys, per channel: [Metal post] "What we're actually optimizing" (keys get
   one scale per channel over a group of tokens) and "Kernel A" (the group of
   channel d is tokens [g*G, min(g*G+G, S)) of that channel).  A ragged last
   group uses its real tokens only; "Three ways to be off by one bit", item 3,
   pads it with copies of the last real token, which leaves min and max --
   and so every result -- unchanged. */
int orc_quantize_keys_meta(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                           int64_t x_bh_stride, int bits, int G,
                           uint32_t *codes, int64_t codes_bh_stride,
                           float *scale, float *zero, int64_t meta_bh_stride,
                           int64_t dst_token,
                           uint16_t *recon, int64_t recon_bh_stride, int fmt, int meta)
{
    if (check_common(BH, S, D, bits, G) != 0) return -1;
    if (meta != ORC_META_F32 && (meta != ORC_META_F16 || fmt != ORC_F16)) return -1;
    if (dst_token < 0 || dst_token % G != 0) return -1;
    const int64_t words = D * bits / 32;
    const int64_t NG = (S + G - 1) / G;
    uint16_t *grp = malloc(sizeof(uint16_t) * (size_t)G);
    uint8_t *q = malloc((size_t)G);
    uint16_t *rec = malloc(sizeof(uint16_t) * (size_t)G);
    if (!grp || !q || !rec) { free(grp); free(q); free(rec); return -1; }

    for (int64_t bh = 0; bh < BH; ++bh) {
        /* the flushed token rows are rewritten in full */
        for (int64_t s = 0; s < S; ++s)
            for (int64_t w = 0; w < words; ++w)
                codes[bh * codes_bh_stride + (dst_token + s) * words + w] = 0u;
        for (int64_t g = 0; g < NG; ++g) {
            const int64_t s0 = g * G;
            const int64_t s1 = (s0 + G < S) ? s0 + G : S;
            const int n = (int)(s1 - s0);
            const int64_t meta_row = dst_token / G + g;
            for (int64_t d = 0; d < D; ++d) {
                for (int i = 0; i < n; ++i)
                    grp[i] = x[bh * x_bh_stride + (s0 + i) * D + d];
                float sc, ze;
                orc_quantize_group_meta(grp, n, bits, fmt, meta, &sc, &ze, q, recon ? rec : NULL);
                scale[bh * meta_bh_stride + meta_row * D + d] = sc;
                zero[bh * meta_bh_stride + meta_row * D + d] = ze;
                for (int i = 0; i < n; ++i) {
                    uint32_t *row = codes + bh * codes_bh_stride + (dst_token + s0 + i) * words;
                    put_code(row, d, bits, q[i]);
                    if (recon) recon[bh * recon_bh_stride + (s0 + i) * D + d] = rec[i];
                }
            }
        }
    }
    free(grp); free(q); free(rec);
    return 0;
}

/* Values, per token: [Metal post] "What we're actually optimizing" (values
   get one scale per token over a group of channels) and "Kernel B" (the
   group of token s is channels [j*G, min(j*G+G, D)) of that token). */
int orc_quantize_values_meta(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                             int64_t x_bh_stride, int bits, int G,
                             uint32_t *codes, int64_t codes_bh_stride,
                             float *scale, float *zero, int64_t meta_bh_stride,
                             int64_t dst_token,
                             uint16_t *recon, int64_t recon_bh_stride, int fmt, int meta)
{
    if (check_common(BH, S, D, bits, G) != 0) return -1;
    if (meta != ORC_META_F32 && (meta != ORC_META_F16 || fmt != ORC_F16)) return -1;
    if (dst_token < 0) return -1;
    const int64_t words = D * bits / 32;
    const int64_t NGD = (D + G - 1) / G;
    uint8_t *q = malloc((size_t)G);
    uint16_t *rec = malloc(sizeof(uint16_t) * (size_t)G);
    if (!q || !rec) { free(q); free(rec); return -1; }

    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t s = 0; s < S; ++s) {
            const uint16_t *xrow = x + bh * x_bh_stride + s * D;
            uint32_t *row = codes + bh * codes_bh_stride + (dst_token + s) * words;
            for (int64_t w = 0; w < words; ++w) row[w] = 0u;
            for (int64_t j = 0; j < NGD; ++j) {
                const int64_t d0 = j * G;
                const int64_t d1 = (d0 + G < D) ? d0 + G : D;
                const int n = (int)(d1 - d0);
                float sc, ze;
                orc_quantize_group_meta(xrow + d0, n, bits, fmt, meta, &sc, &ze, q, recon ? rec : NULL);
                scale[bh * meta_bh_stride + (dst_token + s) * NGD + j] = sc;
                zero[bh * meta_bh_stride + (dst_token + s) * NGD + j] = ze;
                for (int i = 0; i < n; ++i) {
                    put_code(row, d0 + i, bits, q[i]);
                    if (recon) recon[bh * recon_bh_stride + s * D + d0 + i] = rec[i];
                }
            }
        }
    }
    free(q); free(rec);
    return 0;
}

int orc_quantize_keys_fmt(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                          int64_t x_bh_stride, int bits, int G,
                          uint32_t *codes, int64_t codes_bh_stride,
                          float *scale, float *zero, int64_t meta_bh_stride,
                          int64_t dst_token,
                          uint16_t *recon, int64_t recon_bh_stride, int fmt)
{
    return orc_quantize_keys_meta(x, BH, S, D, x_bh_stride, bits, G, codes, codes_bh_stride,
                                  scale, zero, meta_bh_stride, dst_token, recon, recon_bh_stride,
                                  fmt, ORC_META_F32);
}

int orc_quantize_values_fmt(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                            int64_t x_bh_stride, int bits, int G,
                            uint32_t *codes, int64_t codes_bh_stride,
                            float *scale, float *zero, int64_t meta_bh_stride,
                            int64_t dst_token,
                            uint16_t *recon, int64_t recon_bh_stride, int fmt)
{
    return orc_quantize_values_meta(x, BH, S, D, x_bh_stride, bits, G, codes, codes_bh_stride,
                                    scale, zero, meta_bh_stride, dst_token, recon, recon_bh_stride,
                                    fmt, ORC_META_F32);
}

int orc_quantize_keys(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                      int64_t x_bh_stride, int bits, int G,
                      uint32_t *codes, int64_t codes_bh_stride,
                      float *scale, float *zero, int64_t meta_bh_stride,
                      int64_t dst_token,
                      uint16_t *recon, int64_t recon_bh_stride)
{
    return orc_quantize_keys_fmt(x, BH, S, D, x_bh_stride, bits, G, codes, codes_bh_stride,
                                 scale, zero, meta_bh_stride, dst_token, recon, recon_bh_stride,
                                 ORC_F16);
}

int orc_quantize_values(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                        int64_t x_bh_stride, int bits, int G,
                        uint32_t *codes, int64_t codes_bh_stride,
                        float *scale, float *zero, int64_t meta_bh_stride,
                        int64_t dst_token,
                        uint16_t *recon, int64_t recon_bh_stride)
{
    return orc_quantize_values_fmt(x, BH, S, D, x_bh_stride, bits, G, codes, codes_bh_stride,
                                   scale, zero, meta_bh_stride, dst_token, recon, recon_bh_stride,
                                   ORC_F16);
}

static uint32_t get_code(const uint32_t *row_words, int64_t d, int bits)
{
    const int64_t per_word = 32 / bits;
    const int shift = (int)(d % per_word) * bits;
    const uint32_t mask = (bits == 32) ? 0xffffffffu : ((1u << bits) - 1u);
    return (row_words[d / per_word] >> shift) & mask;
}

/* Dequantization, [Metal post] "So why does the kernel ship?" (the packed
   store is expanded back to fp16) with the element rule of
   orc_dequantize_one. */
int orc_dequantize_fmt(int kind, const uint32_t *codes, int64_t codes_bh_stride,
                       const float *scale, const float *zero, int64_t meta_bh_stride,
                       int64_t BH, int64_t D, int bits, int G,
                       int64_t t0, int64_t n,
                       uint16_t *out, int64_t out_bh_stride, int fmt)
{
    if (check_common(BH, n, D, bits, G) != 0) return -1;
    if (t0 < 0 || (kind != ORC_KEYS && kind != ORC_VALUES)) return -1;
    const int64_t words = D * bits / 32;
    const int64_t NGD = (D + G - 1) / G;
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t i = 0; i < n; ++i) {
            const int64_t t = t0 + i;
            const uint32_t *row = codes + bh * codes_bh_stride + t * words;
            for (int64_t d = 0; d < D; ++d) {
                int64_t m;
                if (kind == ORC_KEYS) m = bh * meta_bh_stride + (t / G) * D + d;
                else                  m = bh * meta_bh_stride + t * NGD + d / G;
                out[bh * out_bh_stride + i * D + d] =
                    orc_dequantize_one_fmt(get_code(row, d, bits), scale[m], zero[m], fmt);
            }
        }
    }
    return 0;
}

int orc_dequantize(int kind, const uint32_t *codes, int64_t codes_bh_stride,
                   const float *scale, const float *zero, int64_t meta_bh_stride,
                   int64_t BH, int64_t D, int bits, int G,
                   int64_t t0, int64_t n,
                   uint16_t *out, int64_t out_bh_stride)
{
    return orc_dequantize_fmt(kind, codes, codes_bh_stride, scale, zero, meta_bh_stride, BH, D,
                              bits, G, t0, n, out, out_bh_stride, ORC_F16);
}

/* ------------------------------------------------------------------ */
/* Dequantize-then-attend, the plain definition softmax(q K^T s) V,   */
/* evaluated in double over the fp16 reconstruction of the store      */
/* followed by the fp16 residual window ([Metal post] "What we're     */
/* actually optimizing": the newest tokens stay fp16; [Benchmarks]    */
/* "KV-Cache Kernel Roofline": the fused kernel is measured against   */
/* dequantize + SDPA on the same compressed state).                   */
/* ------------------------------------------------------------------ */

int orc_decode_attend_fmt(const uint16_t *q, int64_t B, int Hq, int Hkv, int64_t D,
                          const uint32_t *k_codes, const float *k_scale, const float *k_zero,
                          const uint32_t *v_codes, const float *v_scale, const float *v_zero,
                          int64_t codes_bh_stride, int64_t k_meta_bh_stride,
                          int64_t v_meta_bh_stride, int bits, int G, int64_t n_quant,
                          const uint16_t *k_res, const uint16_t *v_res,
                          int64_t res_bh_stride, int64_t n_res,
                          double softmax_scale, double *out, int fmt)
{
    const widen_fn widen = widen_of(fmt);
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || n_quant < 0 || n_res < 0) return -1;
    if (n_quant > 0 && check_common(1, n_quant, D, bits, G) != 0) return -1;
    const int64_t N = n_quant + n_res;
    if (N == 0) return -1;                /* softmax over nothing is undefined */
    const int group = Hq / Hkv;
    uint16_t *kq = malloc(sizeof(uint16_t) * (size_t)(n_quant * D + 1));
    uint16_t *vq = malloc(sizeof(uint16_t) * (size_t)(n_quant * D + 1));
    double *kk = malloc(sizeof(double) * (size_t)(N * D));
    double *vv = malloc(sizeof(double) * (size_t)(N * D));
    double *sc = malloc(sizeof(double) * (size_t)N);
    if (!kq || !vq || !kk || !vv || !sc) {
        free(kq); free(vq); free(kk); free(vv); free(sc);
        return -1;
    }
    for (int64_t b = 0; b < B; ++b) {
        for (int kv = 0; kv < Hkv; ++kv) {
            const int64_t bh = b * Hkv + kv;
            /* K-hat and V-hat: the store's 16-bit reconstruction (fp16 or
               bfloat16, `fmt`), then the residual rows, all widened exactly */
            if (n_quant > 0) {
                orc_dequantize_fmt(ORC_KEYS, k_codes + bh * codes_bh_stride, 0,
                                   k_scale + bh * k_meta_bh_stride,
                                   k_zero + bh * k_meta_bh_stride, 0,
                                   1, D, bits, G, 0, n_quant, kq, 0, fmt);
                orc_dequantize_fmt(ORC_VALUES, v_codes + bh * codes_bh_stride, 0,
                                   v_scale + bh * v_meta_bh_stride,
                                   v_zero + bh * v_meta_bh_stride, 0,
                                   1, D, bits, G, 0, n_quant, vq, 0, fmt);
            }
            for (int64_t j = 0; j < N; ++j) {
                for (int64_t d = 0; d < D; ++d) {
                    uint16_t kh, vh;
                    if (j < n_quant) {
                        kh = kq[j * D + d];
                        vh = vq[j * D + d];
                    } else {
                        kh = k_res[bh * res_bh_stride + (j - n_quant) * D + d];
                        vh = v_res[bh * res_bh_stride + (j - n_quant) * D + d];
                    }
                    kk[j * D + d] = (double)widen(kh);
                    vv[j * D + d] = (double)widen(vh);
                }
            }
            for (int h = kv * group; h < (kv + 1) * group; ++h) {
                const uint16_t *qrow = q + (b * Hq + h) * D;
                double m = -INFINITY;
                for (int64_t j = 0; j < N; ++j) {
                    double s = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        s += (double)widen(qrow[d]) * kk[j * D + d];
                    sc[j] = s * softmax_scale;
                    if (sc[j] > m) m = sc[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    sc[j] = exp(sc[j] - m);
                    l += sc[j];
                }
                double *orow = out + (b * Hq + h) * D;
                for (int64_t d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < N; ++j) acc += sc[j] * vv[j * D + d];
                    orow[d] = acc / l;
                }
            }
        }
    }
    free(kq); free(vq); free(kk); free(vv); free(sc);
    return 0;
}

/* [Metal post], "What we're actually optimizing" (the newest R tokens stay
   fp16 and the rest are flushed in a batch) and "The full end-to-end
   record", Generation 1 (flush/layer 512, 2016, 8160 for prompts of 559,
   2059, 8209 tokens with R = G = 32): whole groups of G among the tokens
   older than the newest R. */
int orc_decode_attend(const uint16_t *q, int64_t B, int Hq, int Hkv, int64_t D,
                      const uint32_t *k_codes, const float *k_scale, const float *k_zero,
                      const uint32_t *v_codes, const float *v_scale, const float *v_zero,
                      int64_t codes_bh_stride, int64_t k_meta_bh_stride,
                      int64_t v_meta_bh_stride, int bits, int G, int64_t n_quant,
                      const uint16_t *k_res, const uint16_t *v_res,
                      int64_t res_bh_stride, int64_t n_res,
                      double softmax_scale, double *out)
{
    return orc_decode_attend_fmt(q, B, Hq, Hkv, D, k_codes, k_scale, k_zero, v_codes, v_scale,
                                 v_zero, codes_bh_stride, k_meta_bh_stride, v_meta_bh_stride,
                                 bits, G, n_quant, k_res, v_res, res_bh_stride, n_res,
                                 softmax_scale, out, ORC_F16);
}

int64_t orc_flush_count(int64_t S, int64_t R, int64_t G)
{
    if (S <= R) return 0;
    return ((S - R) / G) * G;
}
