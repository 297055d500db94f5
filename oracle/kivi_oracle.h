/*
 * kivi_oracle.h -- declarations of the CPU oracle for the KIVI flush,
 * dequantize and dequantize-then-attend.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's cpu_baseline leg may load or call this library; the product
 * path never does.  It shares no code, header, table or constant with the
 * HIP library: the only thing the two have in common is the documented
 * byte layout of the packed store, which is the interface under test.
 *
 * Store layout (the pages fix none; this is the reading both sides are
 * written against):
 *   codes  uint32 [BH][cap][D*bits/32]  token-major; the code of channel d
 *          of token t sits in word (t, d / (32/bits)), bits
 *          [bits*(d % (32/bits)), +bits), least significant first.
 *   keys   scale/zero fp32 [BH][cap/G][D]      (one pair per token group
 *          and channel: per-channel quantization)
 *   values scale/zero fp32 [BH][cap][ceil(D/G)] (one pair per token and
 *          channel group: per-token quantization)
 * Strides are in elements of the array they index.
 */
#ifndef KIVI_ORACLE_H
#define KIVI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 <-> binary32, round to nearest even, with subnormals. */
float    orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float f);
void     orc_f16_to_f32_array(const uint16_t *h, float *f, int64_t n);
void     orc_f32_to_f16_array(const float *f, uint16_t *h, int64_t n);

/* bfloat16 <-> binary32 (binary32 with the low 16 fraction bits dropped),
   round to nearest even, with subnormals. */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);
void     orc_bf16_to_f32_array(const uint16_t *h, float *f, int64_t n);
void     orc_f32_to_bf16_array(const float *f, uint16_t *h, int64_t n);

/* 16-bit storage format of inputs and reconstructions for the _fmt calls. */
enum { ORC_F16 = 0, ORC_BF16 = 1 };

/* The calls below without _fmt read and write fp16; their _fmt twins take
   the format as their last (or, for the group, fourth) argument. */
void orc_quantize_group_fmt(const uint16_t *x, int n, int bits, int fmt,
                            float *scale, float *zero, uint8_t *q, uint16_t *recon);
uint16_t orc_dequantize_one_fmt(uint32_t q, float scale, float zero, int fmt);
int orc_quantize_keys_fmt(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                          int64_t x_bh_stride, int bits, int G,
                          uint32_t *codes, int64_t codes_bh_stride,
                          float *scale, float *zero, int64_t meta_bh_stride,
                          int64_t dst_token,
                          uint16_t *recon, int64_t recon_bh_stride, int fmt);
int orc_quantize_values_fmt(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                            int64_t x_bh_stride, int bits, int G,
                            uint32_t *codes, int64_t codes_bh_stride,
                            float *scale, float *zero, int64_t meta_bh_stride,
                            int64_t dst_token,
                            uint16_t *recon, int64_t recon_bh_stride, int fmt);
int orc_dequantize_fmt(int kind, const uint32_t *codes, int64_t codes_bh_stride,
                       const float *scale, const float *zero, int64_t meta_bh_stride,
                       int64_t BH, int64_t D, int bits, int G,
                       int64_t t0, int64_t n,
                       uint16_t *out, int64_t out_bh_stride, int fmt);

/* Storage format of a store's scale and zero for the _meta calls: binary32,
   or binary16 (fp16 inputs only).  The store arrays stay float either way:
   with ORC_META_F16 they hold the binary16 values widened (exactly), and
   the codes and reconstructions are taken with those rounded values. */
enum { ORC_META_F32 = 0, ORC_META_F16 = 1 };

void orc_quantize_group_meta(const uint16_t *x, int n, int bits, int fmt, int meta,
                             float *scale, float *zero, uint8_t *q, uint16_t *recon);
int orc_quantize_keys_meta(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                           int64_t x_bh_stride, int bits, int G,
                           uint32_t *codes, int64_t codes_bh_stride,
                           float *scale, float *zero, int64_t meta_bh_stride,
                           int64_t dst_token,
                           uint16_t *recon, int64_t recon_bh_stride, int fmt, int meta);
int orc_quantize_values_meta(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                             int64_t x_bh_stride, int bits, int G,
                             uint32_t *codes, int64_t codes_bh_stride,
                             float *scale, float *zero, int64_t meta_bh_stride,
                             int64_t dst_token,
                             uint16_t *recon, int64_t recon_bh_stride, int fmt, int meta);

/* One quantization group of n fp16 values.  Writes scale, zero, the n codes
   and the n fp16 reconstructions (recon may be NULL). */
void orc_quantize_group(const uint16_t *x, int n, int bits,
                        float *scale, float *zero, uint8_t *q, uint16_t *recon);

/* Reconstruct one element from its code and its group's scale and zero. */
uint16_t orc_dequantize_one(uint32_t q, float scale, float zero);

/* Per-channel key flush of x[BH][S][D] (row stride x_bh_stride elements per
   bh) into a store at token offset dst_token (a multiple of G).  Returns 0,
   or -1 on an argument it does not support. */
int orc_quantize_keys(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                      int64_t x_bh_stride, int bits, int G,
                      uint32_t *codes, int64_t codes_bh_stride,
                      float *scale, float *zero, int64_t meta_bh_stride,
                      int64_t dst_token,
                      uint16_t *recon, int64_t recon_bh_stride);

/* Per-token value flush, same arguments; dst_token may be any offset. */
int orc_quantize_values(const uint16_t *x, int64_t BH, int64_t S, int64_t D,
                        int64_t x_bh_stride, int bits, int G,
                        uint32_t *codes, int64_t codes_bh_stride,
                        float *scale, float *zero, int64_t meta_bh_stride,
                        int64_t dst_token,
                        uint16_t *recon, int64_t recon_bh_stride);

#define ORC_KEYS   0
#define ORC_VALUES 1

/* fp16 reconstruction of tokens [t0, t0+n) of a store into out[BH][n][D]. */
int orc_dequantize(int kind, const uint32_t *codes, int64_t codes_bh_stride,
                   const float *scale, const float *zero, int64_t meta_bh_stride,
                   int64_t BH, int64_t D, int bits, int G,
                   int64_t t0, int64_t n,
                   uint16_t *out, int64_t out_bh_stride);

/* softmax(q K^T * softmax_scale) V for one new query token per sequence, in
   double precision, over [dequantized store tokens 0..n_quant-1 ; fp16
   residual tokens 0..n_res-1].  q is fp16 [B][Hq][D]; out is double
   [B][Hq][D]; query head h reads kv head h / (Hq/Hkv); store and residual
   rows are indexed by b*Hkv + kv. */
int orc_decode_attend(const uint16_t *q, int64_t B, int Hq, int Hkv, int64_t D,
                      const uint32_t *k_codes, const float *k_scale, const float *k_zero,
                      const uint32_t *v_codes, const float *v_scale, const float *v_zero,
                      int64_t codes_bh_stride, int64_t k_meta_bh_stride,
                      int64_t v_meta_bh_stride, int bits, int G, int64_t n_quant,
                      const uint16_t *k_res, const uint16_t *v_res,
                      int64_t res_bh_stride, int64_t n_res,
                      double softmax_scale, double *out);

/* orc_decode_attend for bfloat16 (fmt ORC_BF16) or fp16 (ORC_F16): q, the
   residual rows and the store's reconstruction are in that format. */
int orc_decode_attend_fmt(const uint16_t *q, int64_t B, int Hq, int Hkv, int64_t D,
                          const uint32_t *k_codes, const float *k_scale, const float *k_zero,
                          const uint32_t *v_codes, const float *v_scale, const float *v_zero,
                          int64_t codes_bh_stride, int64_t k_meta_bh_stride,
                          int64_t v_meta_bh_stride, int bits, int G, int64_t n_quant,
                          const uint16_t *k_res, const uint16_t *v_res,
                          int64_t res_bh_stride, int64_t n_res,
                          double softmax_scale, double *out, int fmt);

/* Number of the oldest tokens of an S-token prefix that a flush quantizes
   when the newest R stay fp16 and only whole groups of G are flushed. */
int64_t orc_flush_count(int64_t S, int64_t R, int64_t G);

#ifdef __cplusplus
}
#endif

#endif
