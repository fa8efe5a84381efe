/* Checks the identity the quantize kernel relies on for the group scale:
 * for L in {3, 15, 255} and a positive finite float x,
 *     RN(x / L) == fma(fma(-q0, L, x), y, q0),  y = RN(1/L), q0 = RN(x * y)
 * (one FMA residual correction of the product with the rounded reciprocal).
 * Usage: scale_division_check [stride]  -- tests every stride-th positive
 * finite bit pattern (stride 1: all of them) plus both ends of every binade.
 * Prints the number of mismatches; exit status 1 if any. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

static uint64_t check(float L, uint32_t bits, uint64_t *n) {
    volatile float one = 1.0f;
    const float y = one / L;
    const float x = from_bits(bits);
    const float want = x / L;
    const float q0 = x * y;
    const float r = fmaf(-q0, L, x);
    const float got = fmaf(r, y, q0);
    (*n)++;
    if (got != want) {
        printf("mismatch L=%g x=%a want=%a got=%a\n", L, x, want, got);
        return 1;
    }
    return 0;
}

int main(int argc, char **argv) {
    const uint64_t stride = argc > 1 ? strtoull(argv[1], NULL, 10) : 1;
    const float Ls[3] = {3.0f, 15.0f, 255.0f};
    uint64_t bad = 0, n = 0;
    for (int li = 0; li < 3; li++) {
        for (uint64_t b = 1; b < 0x7F800000u; b += stride) bad += check(Ls[li], (uint32_t)b, &n);
        for (uint32_t e = 0; e < 255; e++) {           /* binade ends */
            bad += check(Ls[li], (e << 23) | 1u, &n);
            bad += check(Ls[li], (e << 23) | 0x7FFFFFu, &n);
        }
    }
    printf("checked %llu, mismatches %llu\n", (unsigned long long)n, (unsigned long long)bad);
    return bad != 0;
}
