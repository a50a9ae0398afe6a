/* Exhaustive check of the oracle's binary32 -> binary16 rounding against the
 * x86 F16C conversion instruction (vcvtps2ph, round-to-nearest-even immediate),
 * over all 2^32 binary32 bit patterns. NaNs only need to stay NaN (payloads
 * are not part of the rounding rule). Prints the number of mismatches. */
#include <immintrin.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint16_t wqo_f16_bits_from_f32(float f);

int main(void)
{
    unsigned long long bad = 0, nan_bad = 0;
    long long first_bad = -1;
#pragma omp parallel for schedule(static) reduction(+:bad, nan_bad)
    for (long long hi = 0; hi < 65536; ++hi) {
        for (uint32_t lo = 0; lo < 65536; ++lo) {
            const uint32_t u = ((uint32_t)hi << 16) | lo;
            float f;
            memcpy(&f, &u, 4);
            const uint16_t ref = _cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
            const uint16_t got = wqo_f16_bits_from_f32(f);
            const int f_nan = ((u & 0x7F800000u) == 0x7F800000u) && (u & 0x7FFFFFu);
            if (f_nan) {
                const int ok = ((got & 0x7C00u) == 0x7C00u) && (got & 0x3FFu)
                            && ((ref & 0x7C00u) == 0x7C00u) && (ref & 0x3FFu);
                if (!ok) nan_bad++;
            } else if (got != ref) {
                bad++;
#pragma omp critical
                if (first_bad < 0) first_bad = (long long)u;
            }
        }
    }
    printf("mismatches %llu nan_mismatches %llu first 0x%llx\n", bad, nan_bad,
           (unsigned long long)(first_bad < 0 ? 0 : first_bad));
    return (bad || nan_bad) ? 1 : 0;
}
