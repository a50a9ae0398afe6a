/*
 * wq_oracle.c -- CPU oracle for weight-only block-32 int4/int8 matmul.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the tests, the package smoke check and the bench's
 * CPU-baseline leg do. It shares no code, header, table or constant with the
 * HIP path.
 *
 * What it computes (sources: the TinyMOSS-Diarize devpost page, "How we built
 * it": weight-only kernels, FP32 activations, dequantization fused into the
 * matmul; the moss-transcribe-diarize-litert model card, "Files" and "v2
 * decoder": an int4 block-32 decoder, "q4b32"; the soniqo MOSS guide (RU),
 * implementation notes: symmetric linear INT8 block-32 quantization):
 *
 *   y[m,n] = sum_b s[n,b] * sum_{k in block b} q[n,k] * x[m,k]
 *
 * with symmetric codes per block of 32 consecutive k, one binary16 scale per
 * block. The pages do not give the scale rule, rounding or byte layout; the
 * readings used here (documented beside the design) are:
 *   - scale  s32 = amax / Q in fp32 (Q = 7 for int4, 127 for int8),
 *            stored as binary16, round to nearest even, subnormals kept;
 *   - codes  q = clamp(rint_even(w / s16), lo, hi), the division in fp32
 *            against the stored binary16 scale; (lo,hi) = (-8,7) or (-128,127);
 *            a block whose stored scale is zero gets all-zero codes;
 *   - int4 layout: two nibbles per byte, low nibble = even k, two's complement;
 *     int8 layout: one two's-complement byte per code; rows of length K.
 *   - int5 (the soniqo MOSS guide, "Use" and "INT5 vs INT8": INT5 is the MLX
 *     default; the pages give no scale rule, grouping or layout, so the same
 *     symmetric block-32 rule is read for it): Q = 15, codes in [-16, 15], 5-bit
 *     two's complement.
 *     A row of K codes is 5K/8 bytes: first K/2 bytes holding the low 4 bits of
 *     every code (two per byte, low nibble = even k), then K/8 bytes holding
 *     bit 4 of every code (code k in bit k%8 of byte k/8).
 *
 * The matmul is the plain definition over the dequantized weights, evaluated in
 * binary64 with a sequential loop over increasing k. Every product x*q*s is
 * exact in binary64 (24 + 8 + 11 significant bits), so the only error is the
 * summation, bounded by (K-1) * 2^-53 * sum_k |x[m,k]| |w^[n,k]|.
 *
 * Preconditions (not checked here): finite inputs; K a positive multiple of 32;
 * amax / Q representable in binary16 (<= 65504).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (fp32 arithmetic is SSE on x86-64, so every float operation is rounded once).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QBLOCK 32

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 from binary32: round to nearest, ties to even.          */
/* Written from the format definition: a finite binary32 value is            */
/* sig * 2^p with an integer significand; the binary16 quantum for a value   */
/* of binary exponent E is 2^(E-10), but never below 2^-24 (the subnormal    */
/* step). The value is rounded to a multiple of that quantum.                */
/* ------------------------------------------------------------------------ */
uint16_t wqo_f16_bits_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t ebits = (u >> 23) & 0xFFu;
    const uint32_t mbits = u & 0x7FFFFFu;

    if (ebits == 0xFFu)                         /* inf or NaN */
        return (uint16_t)(sign | 0x7C00u | (mbits ? 0x0200u : 0u));
    if (ebits == 0 && mbits == 0)               /* signed zero */
        return sign;

    /* value = sig * 2^p, sig < 2^24 */
    uint32_t sig;
    int p, e_floor;                             /* e_floor = floor(log2 value) */
    if (ebits == 0) {                           /* binary32 subnormal */
        sig = mbits;
        p = -149;
        e_floor = -127;                         /* any value below 2^-126 */
    } else {
        sig = mbits | 0x800000u;
        p = (int)ebits - 127 - 23;
        e_floor = (int)ebits - 127;
    }

    int q = e_floor - 10;                       /* quantum exponent */
    if (q < -24) q = -24;
    const int shift = q - p;                    /* bits of sig dropped */

    uint64_t r;
    if (shift <= 0) {
        r = (uint64_t)sig << (-shift);          /* exact */
    } else if (shift >= 26) {
        r = 0;                                  /* below half a quantum */
    } else {
        const uint64_t s = sig;
        const uint64_t keep = s >> shift;
        const uint64_t rem = s & ((1ull << shift) - 1);
        const uint64_t half = 1ull << (shift - 1);
        r = keep;
        if (rem > half || (rem == half && (keep & 1u)))
            r = keep + 1;
    }

    if (q == -24 && r <= 1024u) {
        /* subnormal result, or the carry into the smallest normal (0x0400) */
        return (uint16_t)(sign | (uint16_t)r);
    }
    while (r >= 2048u) { r >>= 1; q += 1; }     /* carry from rounding: exact */
    const int E = q + 25;                       /* value = r * 2^q, r in [1024,2048) */
    if (E >= 31)
        return (uint16_t)(sign | 0x7C00u);      /* overflow to infinity */
    return (uint16_t)(sign | ((uint32_t)E << 10) | (uint32_t)(r - 1024u));
}

/* binary16 bits to binary64 (exact). */
double wqo_f64_from_f16_bits(uint16_t h)
{
    const int s = (h >> 15) & 1;
    const int E = (h >> 10) & 0x1F;
    const int man = h & 0x3FF;
    double v;
    if (E == 0)
        v = ldexp((double)man, -24);
    else if (E == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), E - 25);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Quantize + encode (the packing step).                                     */
/* w: fp32 [N][K] row-major. q: int4 -> [N][K/2] bytes, int5 -> [N][5K/8],    */
/* int8 -> [N][K] bytes.                                                     */
/* scales: binary16 bits [N][K/32].                                          */
/* ------------------------------------------------------------------------ */
static void quantize_block(const float *w, int bits, int8_t codes[QBLOCK], uint16_t *scale_bits)
{
    const int Qmax = (bits == 4) ? 7 : (bits == 5) ? 15 : 127;
    const int lo = -Qmax - 1;
    const int hi = Qmax;

    /* 1. largest magnitude in the block (exact in fp32) */
    float amax = 0.0f;
    for (int i = 0; i < QBLOCK; ++i) {
        const float a = fabsf(w[i]);
        if (a > amax) amax = a;
    }
    /* 2. fp32 scale, then 3. its binary16 rounding */
    const float s32 = amax / (float)Qmax;
    uint16_t s16 = wqo_f16_bits_from_f32(s32);
    const float s = (float)wqo_f64_from_f16_bits(s16);   /* exact */

    /* 4. a zero (or underflowed) scale stores zero codes */
    if (s == 0.0f) {
        *scale_bits = 0;
        for (int i = 0; i < QBLOCK; ++i) codes[i] = 0;
        return;
    }
    *scale_bits = s16;
    /* 5. codes against the stored scale: fp32 division, round half to even, clamp */
    for (int i = 0; i < QBLOCK; ++i) {
        const float r = w[i] / s;
        float t = rintf(r);                     /* default rounding mode: nearest-even */
        if (t < (float)lo) t = (float)lo;
        if (t > (float)hi) t = (float)hi;
        codes[i] = (int8_t)t;
    }
}

void wqo_quantize(const float *w, int64_t N, int64_t K, int bits, uint8_t *q, uint16_t *scales)
{
    const int64_t nb = K / QBLOCK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            int8_t codes[QBLOCK];
            quantize_block(w + n * K + b * QBLOCK, bits, codes, &scales[n * nb + b]);
            if (bits == 4 || bits == 5) {
                const int64_t row = (bits == 4) ? K / 2 : K / 2 + K / 8;
                uint8_t *dst = q + n * row + b * (QBLOCK / 2);
                for (int j = 0; j < QBLOCK / 2; ++j) {
                    const uint8_t even = (uint8_t)codes[2 * j] & 0x0Fu;
                    const uint8_t odd = (uint8_t)codes[2 * j + 1] & 0x0Fu;
                    dst[j] = (uint8_t)(even | (odd << 4));
                }
                if (bits == 5) {
                    uint8_t *hb = q + n * row + K / 2 + b * (QBLOCK / 8);
                    for (int j = 0; j < QBLOCK / 8; ++j) hb[j] = 0;
                    for (int i = 0; i < QBLOCK; ++i)
                        hb[i / 8] |= (uint8_t)((((uint8_t)codes[i] >> 4) & 1u) << (i % 8));
                }
            } else {
                uint8_t *dst = q + n * K + b * QBLOCK;
                for (int j = 0; j < QBLOCK; ++j) dst[j] = (uint8_t)codes[j];
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Decode one code (two's complement nibble, 5-bit field or byte).           */
/* ------------------------------------------------------------------------ */
static int code_at(const uint8_t *q, int64_t K, int bits, int64_t n, int64_t k)
{
    if (bits == 4) {
        const uint8_t byte = q[n * (K / 2) + k / 2];
        const int t = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        return (t >= 8) ? t - 16 : t;
    }
    if (bits == 5) {
        const uint8_t *row = q + n * (K / 2 + K / 8);
        const uint8_t byte = row[k / 2];
        const int lo4 = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        const int t = lo4 | (((row[K / 2 + k / 8] >> (k % 8)) & 1) << 4);
        return (t >= 16) ? t - 32 : t;
    }
    const uint8_t byte = q[n * K + k];
    return (byte >= 128) ? (int)byte - 256 : (int)byte;
}

void wqo_decode(const uint8_t *q, int64_t N, int64_t K, int bits, int8_t *codes)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (int8_t)code_at(q, K, bits, n, k);
}

/* Dequantized weight w^[n,k] = q[n,k] * s[n, k/32], exact in binary64. */
void wqo_dequant(const uint8_t *q, const uint16_t *scales, int64_t N, int64_t K, int bits, double *w_hat)
{
    const int64_t nb = K / QBLOCK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            w_hat[n * K + k] = (double)code_at(q, K, bits, n, k)
                             * wqo_f64_from_f16_bits(scales[n * nb + k / QBLOCK]);
}

/* ------------------------------------------------------------------------ */
/* Matmul over the dequantized weights, binary64, sequential in k.           */
/* y[m,n] = sum_k x[m,k] * w^[n,k];  absum[m,n] = sum_k |x[m,k]| |w^[n,k]|.   */
/* If x16 != 0, x is first rounded to binary16 (the fp16-activation          */
/* diagnostic reference). absum may be NULL. threads <= 0: runtime default.   */
/* ------------------------------------------------------------------------ */
void wqo_matmul(const float *x, int64_t M, int64_t K, int64_t N, int bits,
                const uint8_t *q, const uint16_t *scales, int x16,
                double *y, double *absum, int threads)
{
    const int64_t nb = K / QBLOCK;
#ifdef _OPENMP
    const int nthr = (threads > 0) ? threads : omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthr)
#else
    (void)threads;
#endif
    for (int64_t n = 0; n < N; ++n) {
        double *wrow = (double *)malloc((size_t)K * sizeof(double));
        for (int64_t k = 0; k < K; ++k)
            wrow[k] = (double)code_at(q, K, bits, n, k)
                    * wqo_f64_from_f16_bits(scales[n * nb + k / QBLOCK]);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, ab = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = (double)x[m * K + k];
                if (x16) xv = wqo_f64_from_f16_bits(wqo_f16_bits_from_f32(x[m * K + k]));
                acc += xv * wrow[k];
                ab += fabs(xv) * fabs(wrow[k]);
            }
            y[m * N + n] = acc;
            if (absum) absum[m * N + n] = ab;
        }
        free(wrow);
    }
}

/* Threads the matmul would use for a given request (reported by the bench). */
int wqo_threads(int threads)
{
#ifdef _OPENMP
    return (threads > 0) ? threads : omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}

/* Bulk binary32 -> binary16 conversion (used by tests for exhaustive checks). */
void wqo_f16_bits_from_f32_array(const float *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = wqo_f16_bits_from_f32(in[i]);
}

/* Bulk binary16 -> binary64 conversion. */
void wqo_f64_from_f16_bits_array(const uint16_t *in, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = wqo_f64_from_f16_bits(in[i]);
}
