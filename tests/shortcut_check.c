/*
 * shortcut_check.c -- CPU check of the two arithmetic shortcuts the HIP flush
 * kernels take in place of the quantizer's IEEE division (test code; it
 * restates the kernels' formulas in C and compares them with the plain
 * binary32 steps of the quantizer, it is not the oracle).
 *
 * The quantizer ([Metal post] "What we're actually optimizing": scale =
 * (max - min) / (2^bits - 1), q = round((x - zero) / scale); "Three ways to
 * be off by one bit": ties to even) divides twice per element group and
 * element.  The kernels replace
 *
 *   1. scale = RN(range / L), L = 2^bits - 1, by three operations:
 *        q0 = RN(range * RN(1/L)); rho = fma(-q0, L, range);
 *        scale = fma(rho, RN(1/L), q0)
 *      claimed equal for every binary32 range in {0} and [2^-24, 2^18) (every
 *      range a group of fp16 values can have lies there).  Checked here for
 *      every one of those ranges, at L = 15 and L = 3.
 *
 *   2. q = rint(RN(t / s)) by q' = rint(RN(t * r)) with r = RN(r0 + r0 *
 *      RN(1 - s * r0)) (one Newton step from a hardware reciprocal r0),
 *      taken only when |RN(t * r) - q'| <= 1/2 - 2^-16; otherwise the kernel
 *      recomputes with the IEEE quotient.  The claim: every taken shortcut
 *      equals the IEEE result, and |RN(t * r) - RN(t / s)| < 2^-17 always.
 *      Checked here for r0 anywhere within +-2 ulp of 1/s (the hardware
 *      reciprocal is specified to 1 ulp), on scales drawn over the whole
 *      range of fp16 groups (binary32 scales, and binary16-rounded scales
 *      for binary16 metadata), with t on both sides of every half-integer
 *      quotient (the near-tie set) and uniformly over [0, range].
 *
 * Build: gcc -O2 -ffp-contract=off (no fast-math), x86-64 SSE arithmetic;
 * fmaf is the correctly rounded fused multiply-add of C99.
 * Output: one line per check, "name checked=N mismatches=M [extra]"; exit
 * status 1 if any mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "must not be built with -ffast-math"
#endif

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* shortcut 1, as the kernel computes it */
static float scale_shortcut(float range, float L)
{
    const float rl = 1.0f / L;
    const float q0 = range * rl;
    const float rho = fmaf(-q0, L, range);
    return fmaf(rho, rl, q0);
}

static int check_scale(int bits)
{
    const float L = (float)((1 << bits) - 1);
    const uint32_t lo = to_bits(0x1p-24f), hi = to_bits(0x1p18f);
    uint64_t checked = 0, bad = 0;
    uint32_t first_bad = 0;
    if (scale_shortcut(0.0f, L) != 0.0f / L || to_bits(scale_shortcut(0.0f, L)) != 0u) {
        ++bad;
        first_bad = 0;
    }
    ++checked;
    for (uint32_t u = lo; u < hi; ++u) {
        const float r = from_bits(u);
        const float want = r / L;
        const float got = scale_shortcut(r, L);
        ++checked;
        if (to_bits(got) != to_bits(want)) {
            if (!bad) first_bad = u;
            ++bad;
        }
    }
    printf("scale bits=%d checked=%llu mismatches=%llu", bits, (unsigned long long)checked,
           (unsigned long long)bad);
    if (bad) printf(" first_range_bits=0x%08x", first_bad);
    printf("\n");
    return bad != 0;
}

/* splitmix64: a small seeded generator for the sampled checks */
static uint64_t sm_state = 0x9E3779B97F4A7C15ull;
static uint64_t sm_next(void)
{
    uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform01(void) { return (double)(sm_next() >> 11) * 0x1p-53; }

/* nearest binary16 value of a binary32 (ties to even), widened back; used
   for the binary16-metadata scales.  Written from the binary16 format:
   1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static float round_to_binary16(float f)
{
    const double a = fabs((double)f);
    if (a == 0.0) return f;
    int e;
    frexp(a, &e);                          /* a = m 2^e, m in [0.5, 1) */
    int q = e - 11;                        /* spacing 2^(e-11) for normals */
    if (q < -24) q = -24;                  /* subnormal spacing */
    const double scaled = ldexp(a, -q);
    double n = floor(scaled);
    const double frac = scaled - n;
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
    const double r = ldexp(n, q);
    return (float)(f < 0 ? -r : r);
}

struct tally {
    uint64_t checked, taken, fallback, wrong, lemma;
    double worst_gap;
};

/* threshold of the near-tie fallback: the kernels' 1/2 - 2^-16; the
   negative control sets it to 1/2 (the shortcut always taken) */
static float near_tie = 0.5f - 0x1p-16f;

/* one (t, s, r0) case of shortcut 2; L is the code bound */
static void one_code(float t, float s, float r0, float L, struct tally *T)
{
    const float e = fmaf(-s, r0, 1.0f);
    const float r = fmaf(r0, e, r0);
    const float y = t * r;
    const float q = rintf(y);
    const float dev = fabsf(y - q);
    const float z = t / s;
    const float want = fminf(fmaxf(rintf(z), 0.0f), L);
    const double gap = fabs((double)y - (double)z);
    ++T->checked;
    if (gap > T->worst_gap) T->worst_gap = gap;
    if (!(gap < 0x1p-17)) ++T->lemma;
    if (dev > near_tie) {
        ++T->fallback;
        return;
    }
    ++T->taken;
    if (q != want) ++T->wrong;
}

/* r0 values within +-2 ulp of 1/s */
static int reciprocals(float s, float out[5])
{
    const float c = 1.0f / s;
    out[0] = c;
    out[1] = nextafterf(c, INFINITY);
    out[2] = nextafterf(c, 0.0f);
    out[3] = nextafterf(out[1], INFINITY);
    out[4] = nextafterf(out[2], 0.0f);
    return 5;
}

static int check_codes(int bits, int meta16, int n_scales, int n_uniform)
{
    const float L = (float)((1 << bits) - 1);
    struct tally T;
    memset(&T, 0, sizeof T);
    for (int i = 0; i < n_scales; ++i) {
        /* a range log-uniform over [2^-24, 2^17], the span of fp16 groups */
        const float range = (float)exp2(-24.0 + 41.0 * uniform01());
        float s = scale_shortcut(range, L);
        if (meta16) {
            s = round_to_binary16(s);
            /* binary16 subnormal scales take the IEEE path in the kernels */
            if (s < 0x1p-14f) continue;
        }
        float r0s[5];
        const int nr = reciprocals(s, r0s);
        /* near-tie set: t within 48 ulps of (k + 1/2) s, both sides */
        for (int k = 0; k < (int)L; ++k) {
            const float mid = (float)(((double)k + 0.5) * (double)s);
            float t = mid;
            for (int u = 0; u < 48; ++u) t = nextafterf(t, 0.0f);
            for (int u = 0; u <= 96; ++u, t = nextafterf(t, INFINITY)) {
                if (t < 0.0f || t > range) continue;
                for (int j = 0; j < nr; ++j) one_code(t, s, r0s[j], L, &T);
            }
        }
        /* uniform t over [0, range] */
        for (int u = 0; u < n_uniform; ++u) {
            const float t = (float)(uniform01() * (double)range);
            for (int j = 0; j < nr; ++j) one_code(t, s, r0s[j], L, &T);
        }
        /* the group's own extremes */
        for (int j = 0; j < nr; ++j) {
            one_code(0.0f, s, r0s[j], L, &T);
            one_code(range, s, r0s[j], L, &T);
        }
    }
    printf("code bits=%d meta=%s checked=%llu mismatches=%llu taken=%llu fallback=%llu "
           "lemma_violations=%llu worst_gap=%.3e\n",
           bits, meta16 ? "f16" : "f32", (unsigned long long)T.checked,
           (unsigned long long)T.wrong, (unsigned long long)T.taken,
           (unsigned long long)T.fallback, (unsigned long long)T.lemma, T.worst_gap);
    return T.wrong != 0 || T.lemma != 0;
}

/* Negative controls: the same checks must catch a plausible mistake.
   (a) the scale without its correction step, RN(range * RN(1/L)), over one
   binade; (b) the reciprocal code with no near-tie fallback. */
static int controls(void)
{
    uint64_t bad_scale = 0;
    for (uint32_t u = 0x3f800000u; u < 0x40000000u; ++u) {
        const float r = from_bits(u);
        if (to_bits(r * (1.0f / 15.0f)) != to_bits(r / 15.0f)) ++bad_scale;
    }
    printf("control scale_without_correction mismatches=%llu\n", (unsigned long long)bad_scale);
    near_tie = 0.5f;
    printf("control ");
    fflush(stdout);
    check_codes(4, 0, 2000, 20);
    near_tie = 0.5f - 0x1p-16f;
    return 0;
}

int main(int argc, char **argv)
{
    int fail = 0;
    const int only_codes = argc > 1 && strcmp(argv[1], "codes") == 0;
    if (!only_codes) {
        fail |= check_scale(4);
        fail |= check_scale(2);
    }
    fail |= check_codes(4, 0, 20000, 200);
    fail |= check_codes(2, 0, 20000, 200);
    fail |= check_codes(4, 1, 20000, 200);
    fail |= check_codes(2, 1, 20000, 200);
    controls();
    return fail;
}
