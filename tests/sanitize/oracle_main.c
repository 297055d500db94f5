/*
 * oracle_main.c -- drives the C oracle (oracle/kivi_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer: every 16-bit pattern
 * through both codecs, flushes of ragged shapes (S not a multiple of G,
 * head_dims whose last value group is short) at both code widths, both
 * input formats and both scale/zero formats into stores of exactly the
 * size the layout needs, dequantize of arbitrary windows, and the attend
 * over store plus residual.  Every buffer is allocated at its exact size, so
 * an index past a shape's end is reported.  Prints "oracle checks passed".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kivi_oracle.h"

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); ++failures; } } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void)
{
    /* xorshift64*: a seeded test-input generator, nothing the oracle computes */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (uint32_t)((rng * 0x2545F4914F6CDD1Dull) >> 32);
}

/* finite 16-bit values of a given format, with some ties, zeros and denormals */
static uint16_t sample(int fmt)
{
    const uint32_t r = next32();
    const float f = ((float)(r % 20001) - 10000.0f) / 997.0f;
    uint16_t h = fmt == ORC_BF16 ? orc_f32_to_bf16(f) : orc_f32_to_f16(f);
    if ((r >> 20) % 37 == 0) h = 0x8000;                 /* -0 */
    if ((r >> 20) % 41 == 0) h = (uint16_t)((r >> 8) & 0x03FF);   /* denormal */
    return h;
}

static void *exact(size_t n) { return malloc(n ? n : 1); }

static void codecs(void)
{
    for (uint32_t h = 0; h < 65536; ++h) {
        const float f = orc_f16_to_f32((uint16_t)h);
        if (!isnan(f)) CHECK(orc_f32_to_f16(f) == h);
        const float b = orc_bf16_to_f32((uint16_t)h);
        if (!isnan(b)) CHECK(orc_f32_to_bf16(b) == h);
    }
    uint16_t h[1000];
    float f[1000];
    uint16_t back[1000];
    for (int i = 0; i < 1000; ++i) h[i] = sample(ORC_F16);
    orc_f16_to_f32_array(h, f, 1000);
    orc_f32_to_f16_array(f, back, 1000);
    CHECK(memcmp(h, back, sizeof h) == 0);
}

static void flush_shapes(void)
{
    const int64_t Ds[] = {16, 48, 96, 128, 256};
    const int Gs[] = {32, 64, 128};
    for (size_t di = 0; di < sizeof Ds / sizeof Ds[0]; ++di)
    for (size_t gi = 0; gi < sizeof Gs / sizeof Gs[0]; ++gi)
    for (int bits = 2; bits <= 4; bits += 2)
    for (int fmt = 0; fmt < 2; ++fmt)
    for (int meta = 0; meta < 2; ++meta) {
        const int64_t D = Ds[di], G = Gs[gi], BH = 3;
        if (meta == ORC_META_F16 && fmt == ORC_BF16) continue;
        if (D % (32 / bits) != 0) continue;
        const int64_t S = 2 * G + 7;                       /* ragged last key group */
        const int64_t cap = S + G;                         /* dst_token = G leaves room */
        const int64_t words = D * bits / 32;
        const int64_t kmeta = (cap + G - 1) / G * D, vmeta = cap * ((D + G - 1) / G);
        uint16_t *x = exact(sizeof(uint16_t) * (size_t)(BH * S * D));
        for (int64_t i = 0; i < BH * S * D; ++i) x[i] = sample(fmt);
        uint32_t *kc = exact(4 * (size_t)(BH * cap * words));
        uint32_t *vc = exact(4 * (size_t)(BH * cap * words));
        float *ks = exact(4 * (size_t)(BH * kmeta)), *kz = exact(4 * (size_t)(BH * kmeta));
        float *vs = exact(4 * (size_t)(BH * vmeta)), *vz = exact(4 * (size_t)(BH * vmeta));
        uint16_t *rec = exact(2 * (size_t)(BH * S * D));
        uint16_t *deq = exact(2 * (size_t)(BH * S * D));
        memset(kc, 0, 4 * (size_t)(BH * cap * words));
        memset(vc, 0, 4 * (size_t)(BH * cap * words));
        memset(ks, 0, 4 * (size_t)(BH * kmeta)); memset(kz, 0, 4 * (size_t)(BH * kmeta));
        memset(vs, 0, 4 * (size_t)(BH * vmeta)); memset(vz, 0, 4 * (size_t)(BH * vmeta));
        CHECK(orc_quantize_keys_meta(x, BH, S, D, S * D, bits, (int)G, kc, cap * words, ks, kz, kmeta,
                                     G, rec, S * D, fmt, meta) == 0);
        CHECK(orc_dequantize_fmt(0, kc, cap * words, ks, kz, kmeta, BH, D, bits, (int)G, G, S, deq,
                                 S * D, fmt) == 0);
        CHECK(memcmp(rec, deq, 2 * (size_t)(BH * S * D)) == 0);
        CHECK(orc_quantize_values_meta(x, BH, S, D, S * D, bits, (int)G, vc, cap * words, vs, vz, vmeta,
                                       cap - S, rec, S * D, fmt, meta) == 0);
        CHECK(orc_dequantize_fmt(1, vc, cap * words, vs, vz, vmeta, BH, D, bits, (int)G, cap - S, S,
                                 deq, S * D, fmt) == 0);
        CHECK(memcmp(rec, deq, 2 * (size_t)(BH * S * D)) == 0);
        /* refused arguments: nothing written, -1 returned */
        CHECK(orc_quantize_keys_meta(x, BH, S, D, S * D, bits, (int)G, kc, cap * words, ks, kz, kmeta,
                                     1, NULL, 0, fmt, meta) == -1);
        CHECK(orc_quantize_keys_meta(x, -1, S, D, S * D, bits, (int)G, kc, cap * words, ks, kz, kmeta,
                                     0, NULL, 0, fmt, meta) == -1);
        CHECK(orc_quantize_values_meta(x, BH, S, D, S * D, 3, (int)G, vc, cap * words, vs, vz, vmeta,
                                       0, NULL, 0, fmt, meta) == -1);
        /* attend: B = 3 sequences of one kv head, Hq = 2, over the value
           window's store tokens [0, cap) with the keys' zero-filled rows,
           and a residual window */
        if (G == 32) {
            const int64_t nr = 5;
            uint16_t *q = exact(2 * (size_t)(BH * 2 * D));
            uint16_t *kr = exact(2 * (size_t)(BH * nr * D));
            uint16_t *vr = exact(2 * (size_t)(BH * nr * D));
            double *out = exact(8 * (size_t)(BH * 2 * D));
            for (int64_t i = 0; i < BH * 2 * D; ++i) q[i] = sample(fmt);
            for (int64_t i = 0; i < BH * nr * D; ++i) { kr[i] = sample(fmt); vr[i] = sample(fmt); }
            if (meta == ORC_META_F32) {
                CHECK(orc_decode_attend_fmt(q, BH, 2, 1, D, kc, ks, kz, vc, vs, vz, cap * words, kmeta,
                                            vmeta, bits, 32, cap, kr, vr, nr * D, nr, 0.125, out,
                                            fmt) == 0);
                for (int64_t i = 0; i < BH * 2 * D; ++i) CHECK(isfinite(out[i]));
                CHECK(orc_decode_attend_fmt(q, BH, 2, 1, D, kc, ks, kz, vc, vs, vz, cap * words, kmeta,
                                            vmeta, bits, 32, 0, kr, vr, nr * D, nr, 0.125, out, fmt) == 0);
                CHECK(orc_decode_attend_fmt(q, BH, 2, 1, D, kc, ks, kz, vc, vs, vz, cap * words, kmeta,
                                            vmeta, bits, 32, 0, kr, vr, nr * D, 0, 0.125, out, fmt) == -1);
            }
            free(q); free(kr); free(vr); free(out);
        }
        free(x); free(kc); free(vc); free(ks); free(kz); free(vs); free(vz); free(rec); free(deq);
    }
    CHECK(orc_flush_count(100, 32, 32) == 64);
    CHECK(orc_flush_count(10, 32, 32) == 0);
}

int main(void)
{
    codecs();
    flush_shapes();
    if (failures) {
        fprintf(stderr, "%d oracle checks failed\n", failures);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
