/*
 * The C oracle (oracle/kla_ref.c) under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py): whole-sequence forwards over all heads and over a head
 * list, ragged sizes, both write-strength modes, the zero-key guard (eps = 0), decode
 * steps, and the argument checks. Built without OpenMP, so every loop runs on the calling
 * thread under the sanitizers. Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kla_ref_forward(const float *q, const float *k, const float *v, const float *log_alpha, const float *eta,
                    double eps, const float *init_state, const int64_t *heads, int n_heads, double *out,
                    double *final_state, int B, int T, int H, int dk, int dv, int nthreads, int beta_mode);
int kla_ref_decode_step(const float *q, const float *k, const float *v, const float *log_alpha, const float *eta,
                        double eps, double *state, const int64_t *heads, int n_heads, double *out, int N, int H,
                        int dk, int dv, int nthreads, int beta_mode);

static int failures = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float uniform_pm1(void) /* splitmix64 step, top 24 bits to [-1, 1) */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (float)((double)(z >> 40) / 8388608.0 - 1.0);
}

static float *fill(size_t n, float scale, float offset)
{
    float *a = (float *)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) a[i] = offset + scale * uniform_pm1();
    return a;
}

static int all_finite(const double *a, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static void forward_case(int B, int T, int H, int dk, int dv, int mode, int zero_keys, double eps)
{
    size_t nt = (size_t)B * T * H;
    float *q = fill(nt * dk, 1.f, 0.f), *k = fill(nt * dk, 1.f, 0.f), *v = fill(nt * dv, 1.f, 0.f);
    float *la = fill(nt, 0.05f, -0.1f), *eta = fill(nt, 0.4f, 0.5f);
    float *s0 = fill((size_t)B * H * dk * dv, 0.3f, 0.f);
    if (zero_keys)
        for (size_t t = 0; t < nt; t += 3)
            for (int i = 0; i < dk; ++i) k[t * dk + i] = 0.f;
    int n = B * H;
    double *out = (double *)malloc(sizeof(double) * (size_t)n * T * dv + 8);
    double *fin = (double *)malloc(sizeof(double) * (size_t)n * dk * dv);
    CHECK(kla_ref_forward(q, k, v, la, eta, eps, s0, NULL, n, out, fin, B, T, H, dk, dv, 1, mode) == 0);
    CHECK(all_finite(out, (size_t)n * T * dv) && all_finite(fin, (size_t)n * dk * dv));
    /* a head list (last head first, then the first) gives those heads' results */
    int64_t heads[2] = {n - 1, 0};
    double *out2 = (double *)malloc(sizeof(double) * 2 * (size_t)T * dv + 8);
    double *fin2 = (double *)malloc(sizeof(double) * 2 * (size_t)dk * dv);
    CHECK(kla_ref_forward(q, k, v, la, eta, eps, NULL, heads, 2, out2, fin2, B, T, H, dk, dv, 1, mode) == 0);
    CHECK(all_finite(out2, 2 * (size_t)T * dv));
    /* a head index out of range is refused */
    int64_t bad[1] = {n};
    CHECK(kla_ref_forward(q, k, v, la, eta, eps, NULL, bad, 1, out2, fin2, B, T, H, dk, dv, 1, mode) == -1);
    free(q); free(k); free(v); free(la); free(eta); free(s0); free(out); free(fin); free(out2); free(fin2);
}

static void decode_case(int N, int H, int dk, int dv, int mode)
{
    size_t nh = (size_t)N * H;
    float *q = fill(nh * dk, 1.f, 0.f), *k = fill(nh * dk, 1.f, 0.f), *v = fill(nh * dv, 1.f, 0.f);
    float *la = fill(nh, 0.05f, -0.1f), *eta = fill(nh, 0.4f, 0.5f);
    for (int i = 0; i < dk; ++i) k[i] = 0.f; /* head 0: zero key */
    double *S = (double *)calloc(nh * dk * dv, sizeof(double));
    double *o = (double *)malloc(sizeof(double) * nh * dv);
    for (int step = 0; step < 3; ++step)
        CHECK(kla_ref_decode_step(q, k, v, la, eta, 0.0, S, NULL, (int)nh, o, N, H, dk, dv, 1, mode) == 0);
    CHECK(all_finite(o, nh * dv) && all_finite(S, nh * dk * dv));
    int64_t heads[1] = {(int64_t)nh - 1};
    CHECK(kla_ref_decode_step(q, k, v, la, eta, 1e-6, S, heads, 1, o, N, H, dk, dv, 1, mode) == 0);
    CHECK(kla_ref_decode_step(q, k, v, la, eta, 1e-6, S, NULL, 3, o, N, H, dk, dv, 1, mode) == -1 || nh == 3);
    free(q); free(k); free(v); free(la); free(eta); free(S); free(o);
}

int main(void)
{
    for (int mode = 0; mode < 2; ++mode) {
        forward_case(1, 1, 1, 8, 8, mode, 0, 1e-6);
        forward_case(2, 37, 3, 16, 8, mode, 0, 1e-6);
        forward_case(1, 70, 2, 8, 16, mode, 1, 0.0); /* zero keys with eps = 0: beta = 0 */
        forward_case(3, 0, 2, 8, 8, mode, 0, 1e-6);  /* T = 0 */
        decode_case(3, 2, 16, 8, mode);
    }
    /* argument checks */
    float x[4] = {0};
    double d[64];
    CHECK(kla_ref_forward(x, x, x, x, x, 0.0, NULL, NULL, 1, d, d, 1, 1, 1, 2, 2, 1, 2) == -1);
    CHECK(kla_ref_forward(x, x, x, x, x, 0.0, NULL, NULL, 5, d, d, 1, 1, 1, 2, 2, 1, 0) == -1);
    CHECK(kla_ref_forward(x, x, x, x, x, 0.0, NULL, NULL, 1, d, d, 1, 1, 0, 2, 2, 1, 0) == -1);
    CHECK(kla_ref_decode_step(x, x, x, x, x, 0.0, d, NULL, 1, d, 1, 1, 2, 2, 1, 7) == -1);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
