/*
 * kda_oracle.c -- plain, slow, sequential fp64 CPU oracle for Kimi Delta
 * Attention (KDA).  TEST INFRASTRUCTURE ONLY: the GPU library never links,
 * includes or calls this file; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark use it.
 *
 * What it computes (source: "Kimi K3 Open Weights: What Is Actually New In Its
 * 2.8 Trillion Parameter Architecture", shivasnotes.com, section 1 "Kimi Delta
 * Attention is a real new kernel family"):
 *
 *   recurrence (the single-head state equation of that section):
 *       S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *       o_t = S_t^T q_t                  (the read uses the UPDATED state)
 *   decay gate (the bounded-sigmoid equation of the same section):
 *       g_t = g_min * sigma(e^A * z_t),  alpha_t = e^{g_t},  g_min = -5
 *
 * S has dk key rows and dv value columns; alpha_t is a vector over the dk key
 * channels and scales S's rows.  Per token the state is first decayed channel
 * by channel, then the old value stored along k is erased (the delta rule),
 * then the new value is written (kimi-k3-course capstone, one-page map,
 * SEQUENCE block).
 *
 * Readings where the page leaves a step open:
 *   - "sigma(e^A z_t)" is read as the logistic function of the product
 *     e^{A_h} * z_t, with one scalar A per head.
 *   - no 1/sqrt(dk) query scale, no output norm or gate: o_t is the raw read.
 *   - beta is used as given (not clamped).
 *
 * Every step below is the literal matrix product in the order written above:
 * fade the rows, erase along k with the faded state, write beta k v^T, read
 * with q.  Nothing is blocked, fused or reordered.  Sums over the key index run
 * in ascending order, so the result does not depend on the thread count.
 *
 * Layouts (row-major, contiguous):
 *   q, k, z : [B, T, H, dk]      v, o : [B, T, H, dv]      beta : [B, T, H]
 *   A       : [H]                S0, S_T : [B, H, dk, dv]  (S0 may be NULL = 0)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_GMIN (-5.0)

/* Bounded decay gate g = g_min * sigma(c * z) with sigma(x) = 1/(1+e^{-x}).
 * For c*z -> -inf, exp(+inf) = inf and 1/inf = 0, so g = -0 and alpha = 1
 * exactly; for c*z -> +inf, g -> g_min. */
static double oracle_gate(double c, double z) {
    return KDA_ORACLE_GMIN / (1.0 + exp(-(c * z)));
}

/* g for n values of z with one head scale A (c = e^A). */
void kda_oracle_gate_f64(int64_t n, const double *z, double A, double *g_out) {
    const double c = exp(A);
    for (int64_t i = 0; i < n; ++i) g_out[i] = oracle_gate(c, z[i]);
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Runs the recurrence for every (b, h).  Returns 0 on success, 1 on a bad
 * argument, 2 when scratch memory cannot be allocated. */
int kda_oracle_f64(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                   const double *q, const double *k, const double *v,
                   const double *z, const double *beta, const double *A,
                   const double *S0, double *o, double *S_T, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return 1;
    if (!A || !S_T) return 1;
    if (T > 0 && (!q || !k || !v || !z || !beta || !o)) return 1;
    const int64_t units = B * H;
    if (units == 0) return 0;
    int failed = 0;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : failed)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t b = u / H, h = u % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        double *w = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !alpha || !w) {
            free(S); free(alpha); free(w);
            failed |= 1;
            continue;
        }
        const double *s0 = S0 ? S0 + u * dk * dv : NULL;
        for (int64_t e = 0; e < dk * dv; ++e) S[e] = s0 ? s0[e] : 0.0;
        const double c = exp(A[h]);

        for (int64_t t = 0; t < T; ++t) {
            const int64_t row = (b * T + t) * H + h;
            const double *qt = q + row * dk;
            const double *kt = k + row * dk;
            const double *zt = z + row * dk;
            const double *vt = v + row * dv;
            const double bt = beta[row];
            double *ot = o + row * dv;

            /* gate: alpha_i = exp(g_min * sigma(c * z_i)) */
            for (int64_t i = 0; i < dk; ++i) alpha[i] = exp(oracle_gate(c, zt[i]));

            /* fade: S <- Diag(alpha) S   (alpha scales key rows) */
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= alpha[i];

            /* erase: S <- (I - beta k k^T) S, via w = S^T k */
            for (int64_t j = 0; j < dv; ++j) w[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) w[j] += kt[i] * S[i * dv + j];
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] -= bt * kt[i] * w[j];

            /* write: S <- S + beta k v^T */
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += bt * kt[i] * vt[j];

            /* read: o = S^T q with the updated state */
            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qt[i];
        }
        memcpy(S_T + u * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S); free(alpha); free(w);
    }
    return failed ? 2 : 0;
}

/*
 * Reverse mode of kda_oracle_f64: the gradient of a scalar loss L through
 * every step above, for the chunked-parallel training form the K3 coverage
 * page lists as the next KDA primitive (nishifamily.com K3 page, innovation
 * table, row "Kimi Delta Attention (linear)").  The pages give no backward
 * formulas; this is the plain definition -- the adjoint of each forward step,
 * taken in reverse order -- written out step by step.
 *
 * Given dO = dL/do [B,T,H,dv] and dST = dL/dS_T [B,H,dk,dv] (NULL = 0), it
 * returns dq, dk, dz [B,T,H,dk], dv [B,T,H,dv], dbeta [B,T,H], dA [H] and
 * dS0 [B,H,dk,dv].  Per (b, h) the forward pass is run once, keeping every
 * state S_0 .. S_T ((T + 1) * dk * dv doubles), then the tokens are walked
 * backwards.  With F = Diag(alpha) S_{t-1}, w = F^T k, E = F - beta k w^T,
 * S_t = E + beta k v^T, o_t = S_t^T q:
 *     read : dq = S_t do;                dS_t += q do^T
 *     write: dbeta += k^T dS_t v;        dk += beta dS_t v;   dv = beta dS_t^T k
 *     erase: dF = dS_t;                  dbeta -= k^T dS_t w; dk -= beta dS_t w;
 *            dw = -beta dS_t^T k;        dF += k dw^T;        dk += F dw
 *     fade : dS_{t-1} = Diag(alpha) dF;  dalpha_i = sum_j dF_ij S_{t-1,ij}
 *     gate : dg = dalpha alpha; dx = dg g_min s (1 - s) with s = sigma(x),
 *            x = c z; dz = c dx; dA += c sum z dx  (c = e^A)
 * dA sums over every b, t and key channel of the head.
 * Returns 0 on success, 1 on a bad argument, 2 when memory is short.
 */
int kda_oracle_bwd_f64(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                       const double *q, const double *k, const double *v,
                       const double *z, const double *beta, const double *A,
                       const double *S0, const double *dO, const double *dST,
                       double *dq, double *dk_out, double *dv_out, double *dz,
                       double *dbeta, double *dA, double *dS0, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return 1;
    if (!A || !dA || !dS0) return 1;
    if (T > 0 && (!q || !k || !v || !z || !beta || !dO || !dq || !dk_out || !dv_out || !dz ||
                  !dbeta))
        return 1;
    const int64_t units = B * H;
    for (int64_t h = 0; h < H; ++h) dA[h] = 0.0;
    if (units == 0) return 0;
    int failed = 0;
    if (nthreads < 1) nthreads = 1;
    const int64_t sd = dk * dv;
    double *dA_unit = (double *)calloc((size_t)units, sizeof(double));
    if (!dA_unit) return 2;

#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : failed)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t b = u / H, h = u % H;
        const double ce = exp(A[h]);   /* e^A */
        /* states S_0 .. S_T (S_0 = initial) */
        double *Sall = (double *)malloc(sizeof(double) * (size_t)((T + 1) * sd));
        double *F = (double *)malloc(sizeof(double) * (size_t)sd);
        double *dS = (double *)malloc(sizeof(double) * (size_t)sd);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        double *dalpha = (double *)malloc(sizeof(double) * (size_t)dk);
        double *w = (double *)malloc(sizeof(double) * (size_t)dv);
        double *dw = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!Sall || !F || !dS || !alpha || !dalpha || !w || !dw) {
            free(Sall); free(F); free(dS); free(alpha); free(dalpha); free(w); free(dw);
            failed |= 1;
            continue;
        }
        const double *s0 = S0 ? S0 + u * sd : NULL;
        for (int64_t e = 0; e < sd; ++e) Sall[e] = s0 ? s0[e] : 0.0;

        /* forward, keeping every state (the same steps as kda_oracle_f64) */
        for (int64_t t = 0; t < T; ++t) {
            const int64_t row = (b * T + t) * H + h;
            const double *kt = k + row * dk, *zt = z + row * dk, *vt = v + row * dv;
            const double bt = beta[row];
            const double *Sp = Sall + t * sd;
            double *Sn = Sall + (t + 1) * sd;
            for (int64_t i = 0; i < dk; ++i) alpha[i] = exp(oracle_gate(ce, zt[i]));
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) Sn[i * dv + j] = alpha[i] * Sp[i * dv + j];
            for (int64_t j = 0; j < dv; ++j) w[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) w[j] += kt[i] * Sn[i * dv + j];
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) Sn[i * dv + j] -= bt * kt[i] * w[j];
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) Sn[i * dv + j] += bt * kt[i] * vt[j];
        }

        /* backward */
        const double *dst = dST ? dST + u * sd : NULL;
        for (int64_t e = 0; e < sd; ++e) dS[e] = dst ? dst[e] : 0.0;
        double dA_acc = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t row = (b * T + t) * H + h;
            const double *qt = q + row * dk, *kt = k + row * dk, *zt = z + row * dk;
            const double *vt = v + row * dv, *dot = dO + row * dv;
            const double bt = beta[row];
            const double *Sp = Sall + t * sd;        /* S_{t-1} */
            const double *St = Sall + (t + 1) * sd;  /* S_t */
            double *dqt = dq + row * dk, *dkt = dk_out + row * dk, *dzt = dz + row * dk;
            double *dvt = dv_out + row * dv;
            double dbt = 0.0;
            /* recompute F and w of this token */
            for (int64_t i = 0; i < dk; ++i) alpha[i] = exp(oracle_gate(ce, zt[i]));
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) F[i * dv + j] = alpha[i] * Sp[i * dv + j];
            for (int64_t j = 0; j < dv; ++j) w[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) w[j] += kt[i] * F[i * dv + j];

            /* read: o = S_t^T q */
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) acc += St[i * dv + j] * dot[j];
                dqt[i] = acc;
            }
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] += qt[i] * dot[j];

            /* write: S_t = E + beta k v^T */
            for (int64_t i = 0; i < dk; ++i) dkt[i] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                double sv = 0.0;
                for (int64_t j = 0; j < dv; ++j) sv += dS[i * dv + j] * vt[j];
                dbt += kt[i] * sv;
                dkt[i] += bt * sv;
            }
            for (int64_t j = 0; j < dv; ++j) {
                double sk = 0.0;
                for (int64_t i = 0; i < dk; ++i) sk += dS[i * dv + j] * kt[i];
                dvt[j] = bt * sk;
                dw[j] = -bt * sk;     /* erase: dw = -beta dE^T k, dE = dS_t */
            }

            /* erase: E = F - beta k w^T, w = F^T k */
            for (int64_t i = 0; i < dk; ++i) {
                double sw = 0.0;
                for (int64_t j = 0; j < dv; ++j) sw += dS[i * dv + j] * w[j];
                dbt -= kt[i] * sw;
                dkt[i] -= bt * sw;
            }
            /* dF = dE + k dw^T (dE = dS_t); dk += F dw */
            for (int64_t i = 0; i < dk; ++i) {
                double fd = 0.0;
                for (int64_t j = 0; j < dv; ++j) fd += F[i * dv + j] * dw[j];
                dkt[i] += fd;
            }
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] += kt[i] * dw[j];

            /* fade: F = Diag(alpha) S_{t-1} */
            for (int64_t i = 0; i < dk; ++i) {
                double da = 0.0;
                for (int64_t j = 0; j < dv; ++j) da += dS[i * dv + j] * Sp[i * dv + j];
                dalpha[i] = da;
                for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] = alpha[i] * dS[i * dv + j];
            }
            /* gate: alpha = exp(g), g = g_min sigma(c z) */
            for (int64_t i = 0; i < dk; ++i) {
                const double x = ce * zt[i];
                const double s = 1.0 / (1.0 + exp(-x));
                const double dg = dalpha[i] * alpha[i];
                const double dx = dg * KDA_ORACLE_GMIN * s * (1.0 - s);
                dzt[i] = ce * dx;
                dA_acc += ce * zt[i] * dx;
            }
            dbeta[row] = dbt;
        }
        memcpy(dS0 + u * sd, dS, sizeof(double) * (size_t)sd);
        dA_unit[u] = dA_acc;
        free(Sall); free(F); free(dS); free(alpha); free(dalpha); free(w); free(dw);
    }
    /* dA: per head, summed over batch entries in ascending order */
    for (int64_t h = 0; h < H; ++h)
        for (int64_t b = 0; b < B; ++b) dA[h] += dA_unit[b * H + h];
    free(dA_unit);
    return failed ? 2 : 0;
}
