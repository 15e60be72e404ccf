/* Exhaustive check of the identity the write kernel uses for the scale:
 *   q0 = x * r,  q1 = fma(fma(-q0, d, x), r, q0)  with r = RN(1 / d)
 * equals the correctly rounded x / d for every non-negative finite binary32 x, for the two
 * level counts d = 15 (4-bit codes) and d = 3 (2-bit codes).  Prints the mismatch count per
 * d; exit status 0 when both are zero.  Build: gcc -O3 -march=native -fopenmp -ffp-contract=off. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint64_t mismatches(float d)
{
    const float r = 1.0f / d;
    uint64_t bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t i = 0; i < 0x7F800000LL; ++i) {
        const uint32_t u = (uint32_t)i;
        float x;
        memcpy(&x, &u, 4);
        const float q0 = x * r;
        const float q1 = fmaf(fmaf(-q0, d, x), r, q0);
        const float ref = x / d;
        uint32_t a, b;
        memcpy(&a, &q1, 4);
        memcpy(&b, &ref, 4);
        bad += a != b;
    }
    return bad;
}

int main(void)
{
    const uint64_t b15 = mismatches(15.0f), b3 = mismatches(3.0f);
    printf("d=15 mismatches=%llu\nd=3 mismatches=%llu\n", (unsigned long long)b15,
           (unsigned long long)b3);
    return (b15 == 0 && b3 == 0) ? 0 : 1;
}
