/*
 * CPU oracle for the KLA forward recurrence: plain C, float64 arithmetic,
 * OpenMP over independent heads.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py load this library. The HIP library never does, and the two
 * share no source.
 *
 * It computes the token-by-token definition of the Kaczmarz Linear Attention
 * (KLA) page: section "Theoretical derivation" (the write projects the decayed
 * state onto S^T k_t = v_t), section "KLA update rule" (beta_t = eta_t /
 * (||k_t||^2 + eps), S_t = S~ + beta_t k_t e_t^T, e_t = v_t - S~^T k_t) and
 * section "Implementation" (the decay gate is kept). Readings where the page is
 * silent: S~ = exp(log_alpha_t) * S_{t-1}; o_t = S_t^T q_t after the write, no
 * query scaling; beta_t = 0 when ||k_t||^2 + eps == 0.
 *
 * beta_mode 1 ("direct") is the Gated DeltaNet baseline the same page sets KLA
 * against (section "Problem statement"): beta_t = eta_t as given, no division
 * by ||k_t||^2 + eps. beta_mode 0 is KLA.
 *
 * Inputs are float32 (bf16 inputs arrive as their exact float32 values); every
 * operation is in double. Layouts: q,k [B,T,H,dk], v [B,T,H,dv], gates [B,T,H],
 * state [B,H,dk,dv] (dv fastest). Outputs are written for a list of heads in
 * compact form: out [n_heads,T,dv], final_state [n_heads,dk,dv].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token for one head. S is dk x dv (row i = key index), updated in place. */
static void token(double *S, const float *q, const float *k, const float *v,
                  double log_alpha, double eta, double eps, int dk, int dv,
                  int beta_mode, double *e, double *o)
{
    double alpha = exp(log_alpha);
    double nk = 0.0;
    for (int i = 0; i < dk; ++i) nk += (double)k[i] * (double)k[i];
    double denom = nk + eps;
    double beta = beta_mode == 1 ? eta : (denom != 0.0 ? eta / denom : 0.0);

    /* S~ = alpha S */
    for (int i = 0; i < dk * dv; ++i) S[i] *= alpha;
    /* e = v - S~^T k */
    for (int j = 0; j < dv; ++j) e[j] = (double)v[j];
    for (int i = 0; i < dk; ++i) {
        double ki = (double)k[i];
        const double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) e[j] -= row[j] * ki;
    }
    /* S = S~ + beta k e^T */
    for (int i = 0; i < dk; ++i) {
        double bk = beta * (double)k[i];
        double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) row[j] += bk * e[j];
    }
    /* o = S^T q */
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        double qi = (double)q[i];
        const double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) o[j] += row[j] * qi;
    }
}

static int threads_or_default(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Whole-sequence forward for the heads listed in `heads` (flat index b*H+h;
 * NULL means all B*H heads in order, n_heads must then be B*H).
 * init_state may be NULL (zeros). Returns 0, or -1 on bad arguments / no memory.
 */
int kla_ref_forward(const float *q, const float *k, const float *v,
                    const float *log_alpha, const float *eta, double eps,
                    const float *init_state, const int64_t *heads, int n_heads,
                    double *out, double *final_state,
                    int B, int T, int H, int dk, int dv, int nthreads, int beta_mode)
{
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || n_heads < 0) return -1;
    if (beta_mode != 0 && beta_mode != 1) return -1;
    if (!heads && n_heads != B * H) return -1;
    int err = 0;
    int nt = threads_or_default(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : err)
    for (int n = 0; n < n_heads; ++n) {
        int64_t flat = heads ? heads[n] : n;
        if (flat < 0 || flat >= (int64_t)B * H) { err |= 1; continue; }
        int64_t b = flat / H, h = flat % H;
        double *S = final_state + (size_t)n * dk * dv;
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!e) { err |= 1; continue; }
        if (init_state) {
            const float *s0 = init_state + (size_t)flat * dk * dv;
            for (int i = 0; i < dk * dv; ++i) S[i] = (double)s0[i];
        } else {
            memset(S, 0, sizeof(double) * (size_t)dk * dv);
        }
        for (int t = 0; t < T; ++t) {
            size_t th = ((size_t)b * T + t) * H + h;
            token(S, q + th * dk, k + th * dk, v + th * dv,
                  (double)log_alpha[th], (double)eta[th], eps, dk, dv, beta_mode, e,
                  out + ((size_t)n * T + t) * dv);
        }
        free(e);
    }
    return err ? -1 : 0;
}

/*
 * One decode step for the listed heads of an [N,H] batch of states.
 * state: [n_heads,dk,dv] doubles for exactly those heads, updated in place.
 * q,k [N,H,dk], v [N,H,dv], gates [N,H] float32. out: [n_heads,dv].
 */
int kla_ref_decode_step(const float *q, const float *k, const float *v,
                        const float *log_alpha, const float *eta, double eps,
                        double *state, const int64_t *heads, int n_heads,
                        double *out, int N, int H, int dk, int dv, int nthreads, int beta_mode)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || n_heads < 0) return -1;
    if (beta_mode != 0 && beta_mode != 1) return -1;
    if (!heads && n_heads != N * H) return -1;
    int err = 0;
    int nt = threads_or_default(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt) reduction(| : err)
    for (int n = 0; n < n_heads; ++n) {
        int64_t flat = heads ? heads[n] : n;
        if (flat < 0 || flat >= (int64_t)N * H) { err |= 1; continue; }
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!e) { err |= 1; continue; }
        token(state + (size_t)n * dk * dv, q + (size_t)flat * dk, k + (size_t)flat * dk,
              v + (size_t)flat * dv, (double)log_alpha[flat], (double)eta[flat], eps,
              dk, dv, beta_mode, e, out + (size_t)n * dv);
        free(e);
    }
    return err ? -1 : 0;
}

int kla_ref_max_threads(void)
{
    return threads_or_default(0);
}
