/* The oracle's C routines under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_sanitize_host.py with -fsanitize=address,undefined and
 * no recovery, so any report ends the run with a non-zero status).
 *
 * Every routine is called over the shapes the tests use and their edges: one
 * block, ragged N, K up to 3072, M up to 33, all three code widths, weights
 * with zero blocks and binary16-subnormal scales (finite, amax / Q <= 65504:
 * the quantizer's stated domain), activations with zeros, subnormals, huge
 * values, inf and NaN (the matmul takes any fp32), and every binary16 bit
 * pattern through the conversions. A few identities are checked on the way
 * (decode(quantize(w)) * scale == dequant; the x16 matmul of binary16-exact x
 * equals the plain one), so the run also fails on a wrong result.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t wqo_f16_bits_from_f32(float f);
double wqo_f64_from_f16_bits(uint16_t h);
void wqo_quantize(const float *w, int64_t N, int64_t K, int bits, uint8_t *q, uint16_t *scales);
void wqo_decode(const uint8_t *q, int64_t N, int64_t K, int bits, int8_t *codes);
void wqo_dequant(const uint8_t *q, const uint16_t *scales, int64_t N, int64_t K, int bits, double *w_hat);
void wqo_matmul(const float *x, int64_t M, int64_t K, int64_t N, int bits, const uint8_t *q,
                const uint16_t *scales, int x16, double *y, double *absum, int threads);
int wqo_threads(int threads);
void wqo_f16_bits_from_f32_array(const float *in, int64_t n, uint16_t *out);
void wqo_f64_from_f16_bits_array(const uint16_t *in, int64_t n, double *out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void)   /* splitmix64 */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

static float normalish(void) { return (float)((uniform() + uniform() + uniform() - 1.5) * 2.0); }

static int failures = 0;
#define CHECK(c, ...)                                  \
    do {                                               \
        if (!(c)) {                                    \
            fprintf(stderr, "check failed: " __VA_ARGS__); \
            fprintf(stderr, "\n");                     \
            failures++;                                \
        }                                              \
    } while (0)

static size_t qrow(int64_t K, int bits) { return (size_t)(bits == 8 ? K : bits == 4 ? K / 2 : K / 2 + K / 8); }

static void one_shape(int64_t N, int64_t K, int bits, int M)
{
    const int Q = bits == 4 ? 7 : bits == 5 ? 15 : 127;
    const int64_t nb = K / 32;
    float *w = malloc(sizeof(float) * (size_t)(N * K));
    for (int64_t i = 0; i < N * K; ++i) w[i] = normalish() * 0.02f;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t b = (int64_t)(next_u64() % (uint64_t)nb);
        memset(w + n * K + b * 32, 0, 32 * sizeof(float));                  /* a zero block */
        const int64_t b2 = (int64_t)(next_u64() % (uint64_t)nb);
        for (int i = 0; i < 32; ++i) w[n * K + b2 * 32 + i] *= 1e-6f;      /* binary16-subnormal scale */
    }
    w[0] = 65504.0f * (float)Q;                                            /* the largest scale */
    uint8_t *q = malloc(qrow(K, bits) * (size_t)N);
    uint16_t *s = malloc(sizeof(uint16_t) * (size_t)(N * nb));
    int8_t *codes = malloc((size_t)(N * K));
    double *wh = malloc(sizeof(double) * (size_t)(N * K));
    wqo_quantize(w, N, K, bits, q, s);
    wqo_decode(q, N, K, bits, codes);
    wqo_dequant(q, s, N, K, bits, wh);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const double ref = (double)codes[n * K + k] * wqo_f64_from_f16_bits(s[n * nb + k / 32]);
            CHECK(wh[n * K + k] == ref, "dequant != decode * scale at bits=%d n=%lld k=%lld", bits,
                  (long long)n, (long long)k);
            CHECK(codes[n * K + k] >= -Q - 1 && codes[n * K + k] <= Q, "code range");
        }
    float *x = malloc(sizeof(float) * (size_t)(M * K));
    for (int64_t i = 0; i < M * K; ++i) x[i] = normalish();
    if (M > 4) {
        x[K + 3] = 0.0f;
        x[K + 4] = 1e-42f;                                                 /* fp32 subnormal */
        x[2 * K + 1] = 3.0e38f;
        x[3 * K] = INFINITY;
        x[4 * K + 7] = NAN;
    }
    double *y = malloc(sizeof(double) * (size_t)(M * N));
    double *y2 = malloc(sizeof(double) * (size_t)(M * N));
    double *ab = malloc(sizeof(double) * (size_t)(M * N));
    wqo_matmul(x, M, K, N, bits, q, s, 0, y, ab, 0);
    wqo_matmul(x, M, K, N, bits, q, s, 1, y2, NULL, 1);
    /* binary16-exact activations: the x16 reference equals the plain one */
    for (int64_t i = 0; i < M * K; ++i) x[i] = (float)((int)(next_u64() % 2001) - 1000) / 64.0f;
    wqo_matmul(x, M, K, N, bits, q, s, 0, y, ab, 2);
    wqo_matmul(x, M, K, N, bits, q, s, 1, y2, NULL, 0);
    for (int64_t i = 0; i < M * N; ++i) CHECK(y[i] == y2[i], "x16 of exact x differs at %lld", (long long)i);
    free(w); free(q); free(s); free(codes); free(wh); free(x); free(y); free(y2); free(ab);
}

int main(void)
{
    /* every binary16 pattern and a sweep of binary32 values through the conversions */
    uint16_t *h = malloc(sizeof(uint16_t) * 65536);
    double *d = malloc(sizeof(double) * 65536);
    for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
    wqo_f64_from_f16_bits_array(h, 65536, d);
    for (int i = 0; i < 65536; ++i) {
        if (isnan(d[i])) continue;
        const uint16_t back = wqo_f16_bits_from_f32((float)d[i]);
        CHECK(back == h[i], "binary16 round trip of 0x%04x", i);
    }
    float *f = malloc(sizeof(float) * 1000000);
    uint16_t *fb = malloc(sizeof(uint16_t) * 1000000);
    for (int i = 0; i < 1000000; ++i) {
        const uint32_t u = (uint32_t)next_u64();
        memcpy(&f[i], &u, 4);
    }
    wqo_f16_bits_from_f32_array(f, 1000000, fb);
    free(h); free(d); free(f); free(fb);

    const int bits_list[3] = {4, 5, 8};
    for (int bi = 0; bi < 3; ++bi) {
        const int bits = bits_list[bi];
        one_shape(1, 32, bits, 1);
        one_shape(3, 96, bits, 2);
        one_shape(257, 1024, bits, 5);
        one_shape(64, 3072, bits, 33);
        one_shape(130, 256, bits, 17);
    }
    CHECK(wqo_threads(3) == 3 && wqo_threads(0) >= 1, "threads");
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitize run: all checks passed\n");
    return 0;
}
