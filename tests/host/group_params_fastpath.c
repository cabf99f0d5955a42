// Host check of the quantizer's division-free decisions (the device helpers
// f16_down_quotient, group_params and quant_codes_b2 in the library's
// internal header), emulated in plain C on random and crafted inputs and
// compared with the IEEE fp32 divisions they replace:
//   * the group scale: largest fp16 <= fp32(num / DEN), taken from
//     m = num * fp32(1 / DEN) unless m is within 8 fp32 ulps of an fp16 value
//     or outside fp16's normal range;
//   * the zero point rint(-lo / D) and the codes rint(v / D) + z, decided from
//     t = fma(v, rd, z + 128.5 + 3 * 2^-16) with rd within 1 ulp of 1 / D
//     (v_rcp_f32's bound, emulated by perturbing the rounded reciprocal by
//     -1, 0 or +1 ulp) unless t's fraction is at most 5 * 2^-16.
// Prints the counts and exits nonzero on any difference.
//     group_params_fastpath [iterations]
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint64_t s64 = 88172645463325252ull;
static uint64_t rnd(void) { s64 ^= s64 << 13; s64 ^= s64 >> 7; s64 ^= s64 << 17; return s64; }
static double urand(void) { return (double)(rnd() >> 11) * (1.0 / 9007199254740992.0); }

static uint16_t f16_down(float d) {   // largest fp16 <= d (d > 0 finite)
    _Float16 h = (_Float16)d;
    uint16_t b;
    memcpy(&b, &h, 2);
    if ((float)h > d) b = (uint16_t)(b - 1);
    return b;
}
static float h2f(uint16_t b) { _Float16 h; memcpy(&h, &b, 2); return (float)h; }

static long check_scale(int den, long iters) {
    const float inv = 1.0f / (float)den;
    long fast = 0, bad = 0;
    for (long it = 0; it < iters; ++it) {
        float num;
        if (it & 1) {
            num = (float)(exp2(-14.0 + 30.0 * urand()) * den);        // log-uniform quotients
        } else {                                                       // crafted: near den * (an fp16 value)
            const uint16_t g = (uint16_t)(0x0400 + rnd() % (0x7BFF - 0x0400));
            const float gv = h2f(g) * (float)den;
            num = bf(fb(gv) + (uint32_t)((int)(rnd() % 41) - 20));
        }
        if (!(num > 0) || isinf(num)) continue;
        const float m = num * inv;
        const uint32_t low = fb(m) & 0x1FFFu;
        if (!(m >= 0x1p-14f && m < 0x1p15f) || low < 8u || low > 0x1FF8u) continue;   // divides
        ++fast;
        if (f16_down(m) != f16_down(num / (float)den)) {
            if (bad++ < 5) printf("scale differs: den %d num %a\n", den, num);
        }
    }
    printf("scale / %d: %ld of %ld decided without the division, %ld differ\n", den, fast, iters, bad);
    return bad;
}

static long check_codes(int Q, long iters) {
    long zfast = 0, cfast = 0, bad = 0;
    for (long it = 0; it < iters; ++it) {
        const float D = h2f((uint16_t)(1 + rnd() % 0x7BFF));
        if (D < 6e-7f) continue;                                       // D >= 1e-5 / 15 always
        const float rd = bf(fb(1.0f / D) + (uint32_t)((int)(rnd() % 3) - 1));
        float mlo;                                                     // -lo >= 0
        if (it & 1) mlo = (float)(urand() * Q * 1.001) * D;
        else mlo = bf(fb(((float)(rnd() % (Q + 1)) + 0.5f) * D) + (uint32_t)((int)(rnd() % 9) - 4));
        if (!(mlo >= 0) || mlo / D > Q * 1.002f) continue;
        const float zr = fminf(fmaxf(rintf(mlo / D), 0.f), (float)Q);
        const uint32_t T = fb(fmaf(mlo, rd, 128.5f + 0x3p-16f));
        if ((T & 0xFFFFu) > 5u) {
            ++zfast;
            if (fminf((float)((T >> 16) & 0xFFu), (float)Q) != zr) {
                if (bad++ < 5) printf("zero point differs: Q %d D %a -lo %a\n", Q, D, mlo);
            }
        }
        float v;                                                       // a value of the group
        if (it & 2) v = -mlo + (float)(urand() * Q) * D;
        else v = bf(fb(((float)(rnd() % (2 * Q + 1)) * 0.5f - 0.5f * Q) * D) + (uint32_t)((int)(rnd() % 9) - 4));
        const float tc = fminf(fmaxf(fmaf(v, rd, zr + (128.5f + 0x3p-16f)), 128.25f), 128.5f + (float)Q);
        const uint32_t Tc = fb(tc);
        if ((Tc & 0xFFFFu) <= 5u) continue;
        ++cfast;
        const float cr = fminf(fmaxf(rintf(v / D) + zr, 0.f), (float)Q);
        if ((float)((Tc >> 16) & 0xFFu) != cr) {
            if (bad++ < 5) printf("code differs: Q %d D %a v %a z %g\n", Q, D, v, zr);
        }
    }
    printf("Q = %d: %ld zero points and %ld codes decided without a division, %ld differ\n", Q, zfast, cfast, bad);
    return bad;
}

int main(int argc, char** argv) {
    const long iters = argc > 1 ? atol(argv[1]) : 4000000;
    long bad = 0;
    bad += check_scale(15, iters) + check_scale(7, iters) + check_scale(3, iters);
    bad += check_codes(15, iters) + check_codes(7, iters);
    return bad ? 1 : 0;
}
