/*
 * CPU oracle for the indexer's key-cache writer: per-token OCP E4M3
 * quantisation of new key vectors, one fp32 scale per token.
 *
 * TEST INFRASTRUCTURE. Like ds4idx_oracle.c, this is the plain reference the
 * HIP writer is checked against; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may build, load or call it. It shares nothing
 * with the HIP library.
 *
 * What the pages fix: the indexer's key cache holds E4M3 codes, and reading
 * codes written in one E4M3 variant (FNUZ) as the other (OCP) is a factor-2
 * scale error (MI300X write-up, "DeepSeek V4 Flash는 단일 AMD MI300X에서
 * 실행됩니다", section on the FP8 format mismatch). They do not print the
 * scale rule or the rounding. The reading taken here is the plainest
 * absmax scaling into the OCP range:
 *
 *   scale[s] = max(amax_s, 2^-126) / 448        (fp32 division)
 *   code[s,d] = E4M3_RNE(clamp(k[s,d] / scale[s], -448, 448))
 *
 * with amax_s = max_d |k[s,d]|, the quotient an IEEE fp32 division, and
 * E4M3_RNE the nearest E4M3FN value with ties to the even code (even last
 * mantissa bit); the sign bit copies the sign of the quotient, so -0.0 and
 * negative values that round to zero give 0x80. The floor 2^-126 keeps the
 * scale positive for an all-zero token. Dequantisation is
 * scale[s] * decode(code[s,d]).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

double ds4o_e4m3_decode(int code); /* ds4idx_oracle.c */

/* The E4M3FN code nearest to x, saturating at +-448, ties to the even code.
 * A linear search over the 127 non-negative finite codes (values ascending):
 * the two candidates that can tie are adjacent codes, and exactly one of them
 * is even. The distances of the two nearest codes are exact in double (x and
 * the code value are within a factor of two of each other, or the code is 0);
 * farther codes are farther by more than any rounding of their distance. */
int ds4o_e4m3_encode(double x)
{
    const int sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a > 448.0)
        a = 448.0;
    int best = 0;
    double best_d = a; /* distance to code 0, value 0 */
    for (int c = 1; c <= 126; c++) {
        const double d = fabs(ds4o_e4m3_decode(c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | best;
}

static float bf16_to_float(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* n key vectors of D values (dtype 0 = fp32, 1 = bf16 bits), row-major.
 * Writes codes [n, D] and scale [n]. Returns 0, or -1 on a bad argument. */
int ds4o_quantize_k(const void *k, int dtype, int64_t n, int D, uint8_t *codes, float *scale)
{
    if (n < 0 || D < 1 || (dtype != 0 && dtype != 1))
        return -1;
    for (int64_t i = 0; i < n; i++) {
        float amax = 0.0f;
        for (int d = 0; d < D; d++) {
            const int64_t j = i * D + d;
            const float v = dtype == 0 ? ((const float *)k)[j] : bf16_to_float(((const uint16_t *)k)[j]);
            const float av = fabsf(v);
            if (av > amax)
                amax = av;
        }
        const float floor_amax = 0x1p-126f;
        const float sc = (amax > floor_amax ? amax : floor_amax) / 448.0f;
        scale[i] = sc;
        for (int d = 0; d < D; d++) {
            const int64_t j = i * D + d;
            const float v = dtype == 0 ? ((const float *)k)[j] : bf16_to_float(((const uint16_t *)k)[j]);
            float qv = v / sc;
            if (qv > 448.0f)
                qv = 448.0f;
            if (qv < -448.0f)
                qv = -448.0f;
            codes[j] = (uint8_t)ds4o_e4m3_encode((double)qv);
        }
    }
    return 0;
}
