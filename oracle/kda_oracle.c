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

/*
 * Backward of kda_oracle_fwd: reverse-mode differentiation of the same
 * recurrence, token by token, in fp64.  The pages give no backward; this is
 * the chain rule applied to the forward above, step by step in reverse:
 *
 *   given dS = dL/dS_t (dL/dS_T from the caller, or 0) and do_t:
 *     dS  += q_t do_t^T               dq_t  = S_t do_t
 *     du   = dS^T k_t                 dk_t  = dS u_t + S'_t dy
 *     dv_t = beta_t du                dbeta_t = du . (v_t - y_t)
 *     dy   = -beta_t du               dS'   = dS + k_t dy^T
 *     da   = rowsum(dS' * S_{t-1})    dS    = Diag(a_t) dS'      (= dL/dS_{t-1})
 *     dg_t = da * a_t * [ -5 <= g_t <= 0 ]   (the clamp passes the gradient
 *                                             inside its closed range)
 *   dS_0 = dS after the first token.
 *
 * The forward states are recomputed: S is kept at every 64th token and the
 * 64 states of a segment are rebuilt from it before that segment's reverse
 * steps.  One work item per (b, h) chain (the key-side gradients sum over
 * all value columns).  Outputs are fp64 in the input layouts; ds0 may be
 * NULL.  Returns 0, -1 for unsupported sizes, -2 if memory runs out.
 */
#define ORACLE_SEG 64

static void forward_token(int K, int V, double* S, const double* a, const double* kk,
                          double bt, const float* vrow, double* y, double* u)
{
    for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= a[i];
    for (int j = 0; j < V; ++j) y[j] = 0.0;
    for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) y[j] += S[(size_t)i * V + j] * kk[i];
    for (int j = 0; j < V; ++j) u[j] = bt * ((double)vrow[j] - y[j]);
    for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) S[(size_t)i * V + j] += kk[i] * u[j];
}

static int bwd_chain(int T, int H, int K, int V, int b, int h,
                     const float* q, const float* k, const float* v, const float* g,
                     const float* beta, const double* s0, const float* d_o, const double* dsT,
                     double* dq, double* dk, double* dv, double* dg, double* dbeta, double* ds0)
{
    const size_t KV = (size_t)K * V;
    const int nseg = (T + ORACLE_SEG - 1) / ORACLE_SEG;
    double* ck = (double*)malloc(sizeof(double) * KV * (size_t)(nseg + 1));   /* S at 64 t */
    double* st = (double*)malloc(sizeof(double) * KV * (ORACLE_SEG + 1));       /* a segment's states */
    double* dS = (double*)malloc(sizeof(double) * KV);
    double* dP = (double*)malloc(sizeof(double) * KV);
    double* a = (double*)malloc(sizeof(double) * 4 * (size_t)K + sizeof(double) * 4 * (size_t)V);
    if (!ck || !st || !dS || !dP || !a) {
        free(ck); free(st); free(dS); free(dP); free(a);
        return -2;
    }
    double* kk = a + K;
    double* qq = kk + K;
    double* da = qq + K;
    double* y = da + K;
    double* u = y + V;
    double* du = u + V;
    double* dy = du + V;
    const size_t chain = ((size_t)b * H + h) * KV;

    /* forward sweep, keeping S at every segment start: ck[m] = S_{64 m},
     * the state before token 64 m */
    double* S = dP;                                    /* running state */
    for (size_t e = 0; e < KV; ++e) S[e] = s0 ? s0[chain + e] : 0.0;
    for (int t = 0; t < T; ++t) {
        if (t % ORACLE_SEG == 0) memcpy(ck + KV * (size_t)(t / ORACLE_SEG), S, sizeof(double) * KV);
        const size_t row = ((size_t)b * T + t) * H + h;
        for (int i = 0; i < K; ++i) {
            a[i] = exp(clamp_log_alpha((double)g[row * K + i]));
            kk[i] = (double)k[row * K + i];
        }
        forward_token(K, V, S, a, kk, (double)beta[row], v + row * V, y, u);
    }

    for (size_t e = 0; e < KV; ++e) dS[e] = dsT ? dsT[chain + e] : 0.0;
    for (int m = nseg - 1; m >= 0; --m) {
        const int t0 = m * ORACLE_SEG;
        const int t1 = (t0 + ORACLE_SEG < T) ? t0 + ORACLE_SEG : T;
        /* st[r] = S_{t0 + r}, rebuilt from the segment's start */
        memcpy(st, ck + KV * (size_t)m, sizeof(double) * KV);
        for (int t = t0; t < t1; ++t) {
            memcpy(st + KV * (size_t)(t - t0 + 1), st + KV * (size_t)(t - t0), sizeof(double) * KV);
            const size_t row = ((size_t)b * T + t) * H + h;
            for (int i = 0; i < K; ++i) {
                a[i] = exp(clamp_log_alpha((double)g[row * K + i]));
                kk[i] = (double)k[row * K + i];
            }
            forward_token(K, V, st + KV * (size_t)(t - t0 + 1), a, kk, (double)beta[row], v + row * V, y, u);
        }
        /* reverse steps of the segment */
        for (int t = t1 - 1; t >= t0; --t) {
            const size_t row = ((size_t)b * T + t) * H + h;
            const double* Sp = st + KV * (size_t)(t - t0);       /* S_{t-1} (before token t) */
            const double* Sc = st + KV * (size_t)(t - t0 + 1);   /* S_t */
            const double bt = (double)beta[row];
            for (int i = 0; i < K; ++i) {
                a[i] = exp(clamp_log_alpha((double)g[row * K + i]));
                kk[i] = (double)k[row * K + i];
                qq[i] = (double)q[row * K + i];
            }
            const float* dor = d_o ? d_o + row * V : NULL;
            /* dS += q do^T; dq = S_t do */
            for (int i = 0; i < K; ++i) {
                double acc = 0.0;
                for (int j = 0; j < V; ++j) {
                    const double doj = dor ? (double)dor[j] : 0.0;
                    dS[(size_t)i * V + j] += qq[i] * doj;
                    acc += Sc[(size_t)i * V + j] * doj;
                }
                dq[row * K + i] = acc;
            }
            /* y = (Diag(a) S_{t-1})^T k, u = beta (v - y) */
            for (int j = 0; j < V; ++j) y[j] = 0.0;
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j) y[j] += a[i] * Sp[(size_t)i * V + j] * kk[i];
            for (int j = 0; j < V; ++j) u[j] = bt * ((double)v[row * V + j] - y[j]);
            /* du = dS^T k */
            for (int j = 0; j < V; ++j) du[j] = 0.0;
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j) du[j] += dS[(size_t)i * V + j] * kk[i];
            double db = 0.0;
            for (int j = 0; j < V; ++j) {
                dv[row * V + j] = bt * du[j];
                db += du[j] * ((double)v[row * V + j] - y[j]);
                dy[j] = -bt * du[j];
            }
            dbeta[row] = db;
            /* dk = dS u + S' dy;  dS' = dS + k dy^T;  da = rowsum(dS' * S_{t-1}) */
            for (int i = 0; i < K; ++i) {
                double acc = 0.0, dai = 0.0;
                for (int j = 0; j < V; ++j) {
                    const size_t e = (size_t)i * V + j;
                    acc += dS[e] * u[j] + a[i] * Sp[e] * dy[j];
                    dP[e] = dS[e] + kk[i] * dy[j];
                    dai += dP[e] * Sp[e];
                }
                dk[row * K + i] = acc;
                const double gi = (double)g[row * K + i];
                dg[row * K + i] = (gi >= -5.0 && gi <= 0.0) ? dai * a[i] : 0.0;
            }
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j) dS[(size_t)i * V + j] = a[i] * dP[(size_t)i * V + j];
        }
    }
    if (ds0)
        for (size_t e = 0; e < KV; ++e) ds0[chain + e] = dS[e];
    free(ck); free(st); free(dS); free(dP); free(a);
    return 0;
}

int kda_oracle_bwd(int B, int T, int H, int K, int V,
                   const float* q, const float* k, const float* v,
                   const float* g, const float* beta, const double* s0,
                   const float* d_o, const double* dsT,
                   double* dq, double* dk, double* dv, double* dg, double* dbeta, double* ds0,
                   int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || K > 512 || V > 512) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(min:rc)
    for (long bh = 0; bh < (long)B * H; ++bh) {
        const int r = bwd_chain(T, H, K, V, (int)(bh / H), (int)(bh % H), q, k, v, g, beta, s0, d_o, dsT,
                                dq, dk, dv, dg, dbeta, ds0);
        if (r < rc) rc = r;
    }
    return rc;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
