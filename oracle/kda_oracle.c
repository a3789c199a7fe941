/*
 * KDA reference oracle: plain, slow, fp64, token by token.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (one independent chain per batch b and head h):
 *
 *   a_t  = exp(min(max(g_t, -5), 0))          per key channel (K values)
 *   S'   = Diag(a_t) S_{t-1}                   forget (decay) step
 *   u_t  = beta_t (v_t - S'^T k_t)             delta-rule error, V values
 *   S_t  = S' + k_t u_t^T                      = (I - beta k k^T) Diag(a) S + beta k v^T
 *   o_t  = S_t^T q_t                           read-out after the update
 *
 * Sources (pages: "Kimi K3 — открытая модель, которая обошла закрытых лидеров
 * рынка", aiblin.ru):
 *   - section "Как хранить миллион токенов в памяти" ("how to keep a million
 *     tokens in memory"): a fixed-size state S replaces the KV cache; every
 *     token rewrites the same state by partly erasing the old content and
 *     writing the new (the delta rule); beta in [0,1] is the write strength,
 *     alpha the forgetting coefficient; alpha is clamped to [e^-5, 1].
 *   - The update formula itself did not survive the pages' HTML extraction
 *     (only its caption, in section "Как распараллелили последовательное
 *     обновление", remains).  The equation above is the standard gated
 *     delta rule with a per-channel diagonal decay that the prose describes;
 *     the readings taken where the pages are silent are: decay before the
 *     erase, read-out from the post-update state, no scale on q, clamp in log
 *     space on both sides, beta not clamped.
 *
 * Parity status: pinned (closed forms, invariants, exact-rational brute
 * force at T <= 8 and hand-derived golden cases; see tests/).
 *
 * Layouts (row-major, token-major as a projection emits them):
 *   q, k, g : [B, T, H, K]        v, o : [B, T, H, V]
 *   beta    : [B, T, H]           s0, sT : [B, H, K, V]
 * Token inputs are fp32 numbers: every bf16 or fp32 input value is
 * represented exactly.  The initial state is fp64 (so a run can resume from
 * another run's fp64 final state), and all arithmetic below is fp64.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_COLS 16   /* value columns handled by one work item */

static double clamp_log_alpha(double g)
{
    /* alpha in [e^-5, 1]  <=>  log alpha in [-5, 0] */
    if (g < -5.0) g = -5.0;
    if (g > 0.0) g = 0.0;
    return g;
}

/*
 * One work item = one (b, h) chain restricted to value columns
 * [c0, c0 + nc).  The recurrence acts on each column of S separately (all
 * column-mixing terms are outer products with the key side), so the columns
 * of one chain can be processed by different work items; the arithmetic on
 * every column is the same, in the same order, as a whole-matrix loop.
 */
static void run_chain(int T, int H, int K, int V, int b, int h, int c0, int nc,
                      const float* q, const float* k, const float* v,
                      const float* g, const float* beta, const double* s0,
                      double* o, double* sT)
{
    double S[ORACLE_MAX_COLS * 512];   /* K x nc, row-major, K <= 512 */
    double a[512], kk[512], qq[512];
    double y[ORACLE_MAX_COLS], u[ORACLE_MAX_COLS];

    for (int i = 0; i < K; ++i)
        for (int j = 0; j < nc; ++j)
            S[i * nc + j] = s0 ? s0[(((size_t)b * H + h) * K + i) * V + c0 + j] : 0.0;

    for (int t = 0; t < T; ++t) {
        const size_t row = ((size_t)b * T + t) * H + h;   /* (b, t, h) */
        const double bt = (double)beta[row];
        for (int i = 0; i < K; ++i) {
            a[i] = exp(clamp_log_alpha((double)g[row * K + i]));
            kk[i] = (double)k[row * K + i];
            qq[i] = (double)q[row * K + i];
        }
        /* S' = Diag(a) S */
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < nc; ++j)
                S[i * nc + j] *= a[i];
        /* y = S'^T k */
        for (int j = 0; j < nc; ++j) y[j] = 0.0;
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < nc; ++j)
                y[j] += S[i * nc + j] * kk[i];
        /* u = beta (v - y) */
        for (int j = 0; j < nc; ++j)
            u[j] = bt * ((double)v[row * V + c0 + j] - y[j]);
        /* S = S' + k u^T */
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < nc; ++j)
                S[i * nc + j] += kk[i] * u[j];
        /* o = S^T q */
        if (o) {
            for (int j = 0; j < nc; ++j) y[j] = 0.0;
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < nc; ++j)
                    y[j] += S[i * nc + j] * qq[i];
            for (int j = 0; j < nc; ++j)
                o[row * V + c0 + j] = y[j];
        }
    }
    if (sT)
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < nc; ++j)
                sT[(((size_t)b * H + h) * K + i) * V + c0 + j] = S[i * nc + j];
}

/*
 * Full forward over all chains.  o and sT may each be NULL (not computed).
 * s0 NULL means a zero initial state.  nthreads <= 0 uses the OpenMP
 * default.  Returns 0, or -1 for unsupported sizes.
 */
int kda_oracle_fwd(int B, int T, int H, int K, int V,
                   const float* q, const float* k, const float* v,
                   const float* g, const float* beta, const double* s0,
                   double* o, double* sT, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || K > 512) return -1;
    const int ncb = (V + ORACLE_MAX_COLS - 1) / ORACLE_MAX_COLS;
    const long items = (long)B * H * ncb;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (long it = 0; it < items; ++it) {
        const int cb = (int)(it % ncb);
        const int h = (int)((it / ncb) % H);
        const int b = (int)(it / ((long)ncb * H));
        const int c0 = cb * ORACLE_MAX_COLS;
        const int nc = (V - c0 < ORACLE_MAX_COLS) ? V - c0 : ORACLE_MAX_COLS;
        run_chain(T, H, K, V, b, h, c0, nc, q, k, v, g, beta, s0, o, sT);
    }
    return 0;
}

/* One decode step for N sequences: the same recurrence with T = 1, state
 * [N, H, K, V] updated in place (fp64), output o [N, H, V]. */
int kda_oracle_step(int N, int H, int K, int V,
                    const float* q, const float* k, const float* v,
                    const float* g, const float* beta, double* state,
                    double* o, int nthreads)
{
    if (N < 0 || H < 0 || K <= 0 || V <= 0 || K > 512) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (long nh = 0; nh < (long)N * H; ++nh) {
        double* S = state + (size_t)nh * K * V;
        const double bt = (double)beta[nh];
        const float* kr = k + (size_t)nh * K;
        const float* qr = q + (size_t)nh * K;
        const float* gr = g + (size_t)nh * K;
        const float* vr = v + (size_t)nh * V;
        for (int i = 0; i < K; ++i) {
            const double a = exp(clamp_log_alpha((double)gr[i]));
            for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= a;
        }
        for (int j = 0; j < V; ++j) {
            double y = 0.0;
            for (int i = 0; i < K; ++i) y += S[(size_t)i * V + j] * (double)kr[i];
            const double u = bt * ((double)vr[j] - y);
            for (int i = 0; i < K; ++i) S[(size_t)i * V + j] += (double)kr[i] * u;
            double z = 0.0;
            for (int i = 0; i < K; ++i) z += S[(size_t)i * V + j] * (double)qr[i];
            o[(size_t)nh * V + j] = z;
        }
    }
    return 0;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
