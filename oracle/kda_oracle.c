/*
 * KDA oracle: plain, slow, fp64 CPU implementation of the Kimi Delta
 * Attention recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes, token by token, for one (sequence, head) at a time:
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t                       (read after the update)
 *
 * with alpha_t = exp(log_alpha_t) per key channel and beta_t a scalar.
 * Sources:
 *   - the KDA state equation: "Kimi K3 核心算子拆解" (devpress.csdn.net),
 *     section 2.2; the same equation in "把注意力换成一块「会遗忘的内存」"
 *     (jokeuncle.github.io), section "第四步:KDA"; and eq. (1)/(3) of
 *     "尝试对Kimi KDA的数学推导&算子实现分析" (hjcheng0602.cn).
 *   - the evaluation order decay -> correction from the decayed state ->
 *     write: "Kimi K3 核心算子拆解", section 2.3 (three-step method).
 *   - readout after the update, o_t = S_t^T q_t: jokeuncle.github.io page,
 *     section "第一步"; "Kimi K3 技术报告解读" (marsggbo.github.io) section 3.2.
 *
 * Steps 2 and 3 of the three-step method are merged into one rank-1 update
 * S <- S + beta k (v - x)^T with x = k^T S (decayed S); this is the same
 * arithmetic the pages write as two rank-1 terms.
 *
 * Layouts (all row-major, last index fastest):
 *   q, k, log_alpha : [T_total, H, dk]      v, o : [T_total, H, dv]
 *   beta            : [T_total, H]          S0, S_T : [N, H, dk, dv]
 *   cu_seqlens      : [N + 1], sequence n owns tokens [cu[n], cu[n+1]).
 * Only value columns [col_begin, col_end) of o and S_T are computed and
 * written (each value column of S evolves on its own, since the transition
 * acts on S from the left); the rest of o / S_T is left untouched.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_OK 0
#define KDA_ORACLE_EINVAL 1
#define KDA_ORACLE_ENOMEM 2

static void run_unit(const double* q, const double* k, const double* v,
                     const double* log_alpha, const double* beta,
                     const double* S0, int64_t t_begin, int64_t t_end,
                     int64_t h, int64_t H, int64_t dk, int64_t dv,
                     int64_t c0, int64_t nc, double* S, double* a, double* x,
                     double* o) {
    /* S is [dk, nc] (columns c0 .. c0+nc-1 of the full state). */
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < nc; ++j)
            S[i * nc + j] = S0 ? S0[i * dv + c0 + j] : 0.0;

    for (int64_t t = t_begin; t < t_end; ++t) {
        const double* kt = k + (t * H + h) * dk;
        const double* qt = q + (t * H + h) * dk;
        const double* vt = v + (t * H + h) * dv;
        const double* lat = log_alpha + (t * H + h) * dk;
        const double bt = beta[t * H + h];

        /* step 1: per-channel decay, S <- Diag(alpha_t) S */
        for (int64_t i = 0; i < dk; ++i) a[i] = exp(lat[i]);
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < nc; ++j) S[i * nc + j] *= a[i];

        /* step 2: what the decayed state returns for key k_t, x = k_t^T S */
        for (int64_t j = 0; j < nc; ++j) x[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < nc; ++j) x[j] += kt[i] * S[i * nc + j];

        /* steps 2+3: erase beta*k x^T and write beta*k v^T */
        for (int64_t i = 0; i < dk; ++i) {
            const double bk = bt * kt[i];
            for (int64_t j = 0; j < nc; ++j)
                S[i * nc + j] += bk * (vt[c0 + j] - x[j]);
        }

        /* readout after the update: o_t = S_t^T q_t */
        double* ot = o + (t * H + h) * dv;
        for (int64_t j = 0; j < nc; ++j) ot[c0 + j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < nc; ++j) ot[c0 + j] += qt[i] * S[i * nc + j];
    }
}

/*
 * Run the recurrence over N packed sequences.  heads/ n_units select a
 * subset of (sequence, head) units: if units != NULL it lists n_units pairs
 * (n, h) flattened as units[2u] = n, units[2u+1] = h; otherwise all N*H
 * units are run.  Returns 0 on success.
 */
int kda_oracle_forward(const double* q, const double* k, const double* v,
                       const double* log_alpha, const double* beta,
                       const double* S0, const int64_t* cu_seqlens,
                       int64_t N, int64_t H, int64_t dk, int64_t dv,
                       int64_t col_begin, int64_t col_end,
                       const int64_t* units, int64_t n_units,
                       double* o, double* S_T, int nthreads) {
    if (!q || !k || !v || !log_alpha || !beta || !cu_seqlens || !o)
        return KDA_ORACLE_EINVAL;
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ORACLE_EINVAL;
    if (col_begin < 0 || col_end > dv || col_begin >= col_end) return KDA_ORACLE_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return KDA_ORACLE_EINVAL;

    const int64_t nc = col_end - col_begin;
    const int64_t total = units ? n_units : N * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel reduction(| : failed)
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)(dk * nc));
        double* a = (double*)malloc(sizeof(double) * (size_t)dk);
        double* x = (double*)malloc(sizeof(double) * (size_t)nc);
        if (!S || !a || !x) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < total; ++u) {
                const int64_t n = units ? units[2 * u] : u / H;
                const int64_t h = units ? units[2 * u + 1] : u % H;
                const double* s0 = S0 ? S0 + (n * H + h) * dk * dv : NULL;
                run_unit(q, k, v, log_alpha, beta, s0, cu_seqlens[n],
                         cu_seqlens[n + 1], h, H, dk, dv, col_begin, nc, S, a,
                         x, o);
                if (S_T) {
                    double* st = S_T + (n * H + h) * dk * dv;
                    for (int64_t i = 0; i < dk; ++i)
                        for (int64_t j = 0; j < nc; ++j)
                            st[i * dv + col_begin + j] = S[i * nc + j];
                }
            }
        }
        free(S);
        free(a);
        free(x);
    }
    return failed ? KDA_ORACLE_ENOMEM : KDA_ORACLE_OK;
}

/*
 * One decode step for B independent requests: the same loop body run once
 * per (request, head) on the carried state S [B, H, dk, dv], which is
 * updated in place; o [B, H, dv].  Inputs are [B, H, d] (one token each).
 */
int kda_oracle_decode_step(const double* q, const double* k, const double* v,
                           const double* log_alpha, const double* beta,
                           double* S, int64_t B, int64_t H, int64_t dk,
                           int64_t dv, double* o, int nthreads) {
    if (!q || !k || !v || !log_alpha || !beta || !S || !o) return KDA_ORACLE_EINVAL;
    if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ORACLE_EINVAL;
    int64_t* cu = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B + 1));
    if (!cu) return KDA_ORACLE_ENOMEM;
    for (int64_t b = 0; b <= B; ++b) cu[b] = b;
    /* each request is a sequence of length 1 whose initial state is S */
    int rc = kda_oracle_forward(q, k, v, log_alpha, beta, S, cu, B, H, dk, dv,
                                0, dv, NULL, 0, o, S, nthreads);
    free(cu);
    return rc;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Backward pass: gradients of a scalar loss L = <dO, o> + <dS_T, S_T> with
 * respect to every input, for the same token loop as kda_oracle_forward.
 * It is the loop's reverse-mode derivative, written out step by step (the
 * backward pass itself is the row "chunk_bwd" the pages list as needed for
 * training in "尝试对Kimi KDA的数学推导&算子实现分析"; the pages give no
 * formula for it, so it is derived here from the forward definition).
 *
 * Forward step t (D = Diag(exp(log_alpha_t))):
 *   S' = D S_{t-1};  x = S'^T k;  u = v - x;  S_t = S' + beta k u^T;
 *   o_t = S_t^T q.
 * Reverse step t, with G = dL/dS_t coming from later steps:
 *   dq_t   = S_t dO_t
 *   G     += q dO_t^T                      (the readout at t)
 *   w      = G^T k                         (dv-vector)
 *   dbeta_t = k^T G u
 *   dv_t   = beta w
 *   dk_t   = beta G u - beta S' w          (direct term, then through x)
 *   dS'    = G - beta k w^T
 *   dlog_alpha_t[i] = sum_j dS'[i][j] S'[i][j]
 *   G      = D dS'                         (= dL/dS_{t-1})
 * and dS0 = G after the first token.  States S_{t-1} are recomputed from
 * checkpoints taken every CK tokens in a first forward sweep; the
 * recomputation repeats the same fp64 operations, so the states are the
 * ones the forward loop produces.
 */
#define KDA_ORACLE_CK 64

static void fwd_token(const double* qt, const double* kt, const double* vt,
                      const double* lat, double bt, int64_t dk, int64_t dv,
                      double* S, double* a, double* x) {
    (void)qt;
    for (int64_t i = 0; i < dk; ++i) a[i] = exp(lat[i]);
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a[i];
    for (int64_t j = 0; j < dv; ++j) x[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) x[j] += kt[i] * S[i * dv + j];
    for (int64_t i = 0; i < dk; ++i) {
        const double bk = bt * kt[i];
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += bk * (vt[j] - x[j]);
    }
}

typedef struct {
    double *ck, *blk, *Sd, *St, *G, *a, *x, *u, *w;
} bwd_scratch;

static void bwd_unit(const double* q, const double* k, const double* v,
                     const double* log_alpha, const double* beta,
                     const double* S0, const double* dO, const double* dST,
                     int64_t t0, int64_t t1, int64_t h, int64_t H, int64_t dk,
                     int64_t dv, double* dq, double* dkk, double* dvv,
                     double* dla, double* dbeta, double* dS0, bwd_scratch* w) {
    const int64_t sz = dk * dv, L = t1 - t0;
    const int64_t nck = (L + KDA_ORACLE_CK - 1) / KDA_ORACLE_CK;
    double* S = w->blk;   /* running state for the sweeps */
    for (int64_t e = 0; e < sz; ++e) S[e] = S0 ? S0[e] : 0.0;
    /* sweep 1: checkpoints of the state before tokens t0 + c * CK */
    for (int64_t t = t0; t < t1; ++t) {
        if ((t - t0) % KDA_ORACLE_CK == 0)
            memcpy(w->ck + ((t - t0) / KDA_ORACLE_CK) * sz, S, sizeof(double) * sz);
        const int64_t r = t * H + h;
        fwd_token(q + r * dk, k + r * dk, v + r * dv, log_alpha + r * dk,
                  beta[r], dk, dv, S, w->a, w->x);
    }
    for (int64_t e = 0; e < sz; ++e) w->G[e] = dST ? dST[e] : 0.0;
    for (int64_t c = nck - 1; c >= 0; --c) {
        const int64_t b0 = t0 + c * KDA_ORACLE_CK;
        const int64_t b1 = b0 + KDA_ORACLE_CK < t1 ? b0 + KDA_ORACLE_CK : t1;
        /* states before each token of the block: blk[(t - b0) * sz] = S_{t-1} */
        memcpy(w->blk, w->ck + c * sz, sizeof(double) * sz);
        for (int64_t t = b0; t + 1 < b1; ++t) {
            double* nxt = w->blk + (t - b0 + 1) * sz;
            memcpy(nxt, w->blk + (t - b0) * sz, sizeof(double) * sz);
            const int64_t r = t * H + h;
            fwd_token(q + r * dk, k + r * dk, v + r * dv, log_alpha + r * dk,
                      beta[r], dk, dv, nxt, w->a, w->x);
        }
        for (int64_t t = b1 - 1; t >= b0; --t) {
            const int64_t r = t * H + h;
            const double* Sp = w->blk + (t - b0) * sz;
            const double *qt = q + r * dk, *kt = k + r * dk, *vt = v + r * dv;
            const double *lat = log_alpha + r * dk, *dot = dO + r * dv;
            const double bt = beta[r];
            double* G = w->G;
            /* recompute S' = D S_{t-1}, u = v - S'^T k, S_t = S' + beta k u^T */
            for (int64_t i = 0; i < dk; ++i) w->a[i] = exp(lat[i]);
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) w->Sd[i * dv + j] = w->a[i] * Sp[i * dv + j];
            for (int64_t j = 0; j < dv; ++j) w->u[j] = vt[j];
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) w->u[j] -= kt[i] * w->Sd[i * dv + j];
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    w->St[i * dv + j] = w->Sd[i * dv + j] + bt * kt[i] * w->u[j];
            /* dq_t = S_t dO_t */
            for (int64_t i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < dv; ++j) s += w->St[i * dv + j] * dot[j];
                dq[r * dk + i] = s;
            }
            /* G += q dO^T */
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) G[i * dv + j] += qt[i] * dot[j];
            /* w = G^T k, dbeta = k^T G u, dv = beta w */
            for (int64_t j = 0; j < dv; ++j) w->w[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) w->w[j] += G[i * dv + j] * kt[i];
            double db = 0.0;
            for (int64_t j = 0; j < dv; ++j) db += w->w[j] * w->u[j];
            dbeta[r] = db;
            for (int64_t j = 0; j < dv; ++j) dvv[r * dv + j] = bt * w->w[j];
            /* dk = beta (G u - S' w) */
            for (int64_t i = 0; i < dk; ++i) {
                double s1 = 0.0, s2 = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    s1 += G[i * dv + j] * w->u[j];
                    s2 += w->Sd[i * dv + j] * w->w[j];
                }
                dkk[r * dk + i] = bt * (s1 - s2);
            }
            /* dS' = G - beta k w^T; dlog_alpha = rowsum(dS' * S'); G = D dS' */
            for (int64_t i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    const double g = G[i * dv + j] - bt * kt[i] * w->w[j];
                    s += g * w->Sd[i * dv + j];
                    G[i * dv + j] = w->a[i] * g;
                }
                dla[r * dk + i] = s;
            }
        }
    }
    if (dS0) memcpy(dS0, w->G, sizeof(double) * sz);
}

/*
 * Gradients for N packed sequences (layouts as kda_oracle_forward; dO like o,
 * dS_T like S_T, may be NULL = zero).  Outputs dq, dk, dlog_alpha [T, H, dk],
 * dv [T, H, dv], dbeta [T, H], dS0 [N, H, dk, dv] (may be NULL).  units as in
 * kda_oracle_forward (rows of units not listed are left untouched).
 */
int kda_oracle_backward(const double* q, const double* k, const double* v,
                        const double* log_alpha, const double* beta,
                        const double* S0, const int64_t* cu_seqlens,
                        int64_t N, int64_t H, int64_t dk, int64_t dv,
                        const double* dO, const double* dS_T,
                        const int64_t* units, int64_t n_units,
                        double* dq, double* dkk, double* dvv, double* dla,
                        double* dbeta, double* dS0, int nthreads) {
    if (!q || !k || !v || !log_alpha || !beta || !cu_seqlens || !dO || !dq ||
        !dkk || !dvv || !dla || !dbeta)
        return KDA_ORACLE_EINVAL;
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ORACLE_EINVAL;
    int64_t maxL = 0;
    for (int64_t n = 0; n < N; ++n) {
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return KDA_ORACLE_EINVAL;
        if (cu_seqlens[n + 1] - cu_seqlens[n] > maxL) maxL = cu_seqlens[n + 1] - cu_seqlens[n];
    }
    const int64_t sz = dk * dv;
    const int64_t nck = (maxL + KDA_ORACLE_CK - 1) / KDA_ORACLE_CK + 1;
    const int64_t total = units ? n_units : N * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : failed)
    {
        bwd_scratch w;
        w.ck = (double*)malloc(sizeof(double) * (size_t)(nck * sz));
        w.blk = (double*)malloc(sizeof(double) * (size_t)(KDA_ORACLE_CK * sz));
        w.Sd = (double*)malloc(sizeof(double) * (size_t)sz);
        w.St = (double*)malloc(sizeof(double) * (size_t)sz);
        w.G = (double*)malloc(sizeof(double) * (size_t)sz);
        w.a = (double*)malloc(sizeof(double) * (size_t)dk);
        w.x = (double*)malloc(sizeof(double) * (size_t)dv);
        w.u = (double*)malloc(sizeof(double) * (size_t)dv);
        w.w = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!w.ck || !w.blk || !w.Sd || !w.St || !w.G || !w.a || !w.x || !w.u || !w.w) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t un = 0; un < total; ++un) {
                const int64_t n = units ? units[2 * un] : un / H;
                const int64_t h = units ? units[2 * un + 1] : un % H;
                const int64_t off = (n * H + h) * sz;
                bwd_unit(q, k, v, log_alpha, beta, S0 ? S0 + off : NULL, dO,
                         dS_T ? dS_T + off : NULL, cu_seqlens[n], cu_seqlens[n + 1],
                         h, H, dk, dv, dq, dkk, dvv, dla, dbeta,
                         dS0 ? dS0 + off : NULL, &w);
            }
        }
        free(w.ck); free(w.blk); free(w.Sd); free(w.St); free(w.G);
        free(w.a); free(w.x); free(w.u); free(w.w);
    }
    return failed ? KDA_ORACLE_ENOMEM : KDA_ORACLE_OK;
}
