/* Host check of the division-free quotient of the E4M3 row quantization.
 *
 * The kernels take x / s from r = fl(1/s), q1 = fl(x r) and one correction
 * by the exact residual, q = fl(q1 + fl(x - q1 s) r) (fused multiply-adds),
 * with the sign of x.  For every positive finite bf16 row maximum a (every
 * stride-th one), s = max(fl(a / 448), 1e-8), and every bf16 x with
 * |x| <= a, this compares the E4M3 code (round to nearest even, saturating
 * at 448) of clamp(q) with that of clamp(fl(x / s)).  Prints the pair count
 * and the number of differing codes; exits 1 if any differ.
 * Build: gcc -O2 -ffp-contract=off row_quotient_check.c -lm */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bf16(uint32_t b) {
    uint32_t u = b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* E4M3 (no infinities, 448 largest) of f with |f| <= 448, round to nearest even */
static int e4m3_code(float f) {
    const int sign = signbit(f) ? 0x80 : 0;
    const float a = fabsf(f);
    if (a < 0x1p-6f) return sign | (int)nearbyintf(a * 0x1p9f); /* subnormals; 8 is 2^-6 */
    int e;
    const float m = frexpf(a, &e); /* a = m 2^e, m in [0.5, 1) */
    int frac = (int)nearbyintf((2.0f * m - 1.0f) * 8.0f);
    int ex = e - 1 + 7;
    if (frac == 8) { frac = 0; ++ex; }
    return sign | (ex << 3) | frac;
}

static float clamp448(float q) { return fminf(fmaxf(q, -448.0f), 448.0f); }

int main(int argc, char** argv) {
    const int stride = argc > 1 ? atoi(argv[1]) : 1;
    long pairs = 0, differ = 0;
    for (uint32_t ab = 1; ab < 0x7F80u; ab += (uint32_t)stride) {
        const float amax = from_bf16(ab);
        float s = amax / 448.0f;
        if (s < 1e-8f) s = 1e-8f;
        const float r = 1.0f / s;
        for (uint32_t xb = 0; xb < 0x10000u; ++xb) {
            const float x = from_bf16(xb);
            if (!(fabsf(x) <= amax)) continue;
            ++pairs;
            const float exact = clamp448(x / s);
            const float q1 = x * r;
            const float fast = clamp448(copysignf(fmaf(fmaf(-q1, s, x), r, q1), x));
            if (bits(fast) != bits(exact) && e4m3_code(fast) != e4m3_code(exact)) {
                if (differ < 5) printf("differ: a=%a x=%a s=%a exact=%a fast=%a\n", amax, x, s, exact, fast);
                ++differ;
            }
        }
    }
    printf("pairs %ld differing codes %ld\n", pairs, differ);
    return differ ? 1 : 0;
}
