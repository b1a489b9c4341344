/*
 * TEST INFRASTRUCTURE ONLY -- the fp64 CPU oracle for causal kernelized linear
 * attention and the delta-rule fast-weight memory.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  The product path (the HIP library) never links, calls or
 * includes anything here, and this file includes nothing from it.
 *
 * Every function is the plain sequential token recurrence in double
 * precision, one (batch, head) pair at a time, written from these pages:
 *
 *   [LinearMem]  "AIGC 基本功｜线性、循环与记忆架构-LinearMem" (jefxiong.cn)
 *   [LA-SSM]     "线性注意力与 SSM:两条技术路线的完整推导" (ggaaooppeenngg.github.io)
 *   [Recurrence] "手撕：递推与记忆模型" (wineandchord.com)
 *
 * Layouts (all row-major, contiguous, host memory, caller-owned):
 *   q, k   [B][H][T][dk]      v, o  [B][H][T][dv]      beta [B][H][T]
 *   S      [B][H][dk][dv]     (key-first, as [LinearMem] §03 defines S_t)
 *   z      [B][H][dk]
 * A NULL S0 / z0 means a zero initial state.  A NULL S_out / z_out means the
 * final state is not returned.  Nothing is allocated that outlives a call.
 *
 * Parity pins: every function here is checked in tests/ against values the
 * pages print, brute-force forms and closed-form invariants (see the module
 * docstring of oracle/__init__.py for the list).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_PHI_ELU1 0     /* phi(u) = u + 1 for u > 0, exp(u) otherwise */
#define ORACLE_PHI_IDENTITY 1 /* phi(u) = u (plain outer-product memory)    */

/* [LinearMem] §03 "从检索权重开始": the elementwise ELU+1 feature map, with
 * the two branches exactly as the page states them (u > 0 -> u + 1,
 * u <= 0 -> exp(u)).  Both branches give 1 at u = 0. */
static double phi_elu1(double u) { return u > 0.0 ? u + 1.0 : exp(u); }

static double feature(double u, int mode) {
    return mode == ORACLE_PHI_IDENTITY ? u : phi_elu1(u);
}

/*
 * Normalized causal linear attention, write-then-read.
 *
 * [LinearMem] §03 "把历史和移到 query 外面": S_t = S_{t-1} + phi(k_t) v_t^T,
 * z_t = z_{t-1} + phi(k_t), S_0 = 0, z_0 = 0, and the read-out
 * o_t^T = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps).  The same section fixes the
 * order: the current token is written before the current query reads.
 * [LinearMem] §04 shows the same loop in NumPy (state kept in float64).
 *
 * Test-only modes reproduce the additive memory of the worked examples:
 *   feature   = ORACLE_PHI_IDENTITY drops the feature map,
 *   normalize = 0 returns the raw read phi(q_t)^T S_t (no z, no eps).
 * With S0/z0 given, the same recurrence continues from them (an initial
 * state is handed in and the final one returned, [Recurrence] "Selective
 * scan" / "Delta-rule fast weight").
 */
void la_ref_forward(const double* q, const double* k, const double* v,
                    const double* S0, const double* z0,
                    double* o, double* S_out, double* z_out,
                    int B, int H, int T, int dk, int dv, double eps,
                    int feature_mode, int normalize) {
    const long heads = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < heads; ++h) {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* z = (double*)malloc(sizeof(double) * (size_t)dk);
        double* fk = (double*)malloc(sizeof(double) * (size_t)dk);
        double* fq = (double*)malloc(sizeof(double) * (size_t)dk);
        for (long i = 0; i < (long)dk * dv; ++i) S[i] = S0 ? S0[h * dk * dv + i] : 0.0;
        for (int i = 0; i < dk; ++i) z[i] = z0 ? z0[h * dk + i] : 0.0;
        const double* qh = q + h * (long)T * dk;
        const double* kh = k + h * (long)T * dk;
        const double* vh = v + h * (long)T * dv;
        double* oh = o + h * (long)T * dv;
        for (int t = 0; t < T; ++t) {
            for (int i = 0; i < dk; ++i) {
                fk[i] = feature(kh[(long)t * dk + i], feature_mode);
                fq[i] = feature(qh[(long)t * dk + i], feature_mode);
            }
            /* write: S += phi(k_t) v_t^T, z += phi(k_t) */
            for (int i = 0; i < dk; ++i) {
                for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += fk[i] * vh[(long)t * dv + j];
                z[i] += fk[i];
            }
            /* read: phi(q_t)^T S_t / (phi(q_t)^T z_t + eps) */
            double den = 0.0;
            for (int i = 0; i < dk; ++i) den += fq[i] * z[i];
            den += eps;
            for (int j = 0; j < dv; ++j) {
                double num = 0.0;
                for (int i = 0; i < dk; ++i) num += fq[i] * S[(long)i * dv + j];
                oh[(long)t * dv + j] = normalize ? num / den : num;
            }
        }
        if (S_out) memcpy(S_out + h * (long)dk * dv, S, sizeof(double) * (size_t)dk * dv);
        if (z_out) memcpy(z_out + h * (long)dk, z, sizeof(double) * (size_t)dk);
        free(S); free(z); free(fk); free(fq);
    }
}

/*
 * Delta-rule fast-weight memory with an optional forgetting gate, write then
 * read.
 *
 * [LinearMem] §03 "从累加改成纠错" and [Recurrence] "Delta-rule fast weight":
 * the write is S_t = S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T, the
 * correction being the new value minus what the memory predicts for k_t.
 * The same §03 then adds a forgetting coefficient alpha_t applied to the old
 * state BEFORE the correction is computed (Gated DeltaNet's rule):
 *   decayed = alpha_t S_{t-1},  u_t = v_t - decayed^T k_t,
 *   S_t = decayed + beta_t k_t u_t^T,
 * with the page's warning that the order (decay first, then the error) is
 * part of the rule.  alpha == NULL means alpha_t = 1 (the plain delta rule).
 * The per-token read o_t = S_t^T q_t (after the write) is this oracle's
 * reading: the pages print no sequence of query reads for this rule.
 * pred (optional, [B][H][T][dv]) receives the prediction decayed^T k_t made
 * before each write: the "read" sequence of [Recurrence] "Delta-rule fast
 * weight", which reads first and then writes with the error.
 */
static void delta_gated_forward(const double* q, const double* k, const double* v,
                                const double* beta, const double* alpha, const double* S0,
                                double* o, double* S_out, double* pred_out,
                                int B, int H, int T, int dk, int dv) {
    const long heads = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < heads; ++h) {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        for (long i = 0; i < (long)dk * dv; ++i) S[i] = S0 ? S0[h * dk * dv + i] : 0.0;
        const double* qh = q + h * (long)T * dk;
        const double* kh = k + h * (long)T * dk;
        const double* vh = v + h * (long)T * dv;
        const double* bh = beta + h * (long)T;
        const double* ah = alpha ? alpha + h * (long)T : NULL;
        double* oh = o + h * (long)T * dv;
        for (int t = 0; t < T; ++t) {
            const double* kt = kh + (long)t * dk;
            /* forget first: the correction is taken against the decayed state */
            if (ah)
                for (long i = 0; i < (long)dk * dv; ++i) S[i] *= ah[t];
            /* correction u = v_t - S^T k_t (new value minus the prediction) */
            for (int j = 0; j < dv; ++j) {
                double pred = 0.0;
                for (int i = 0; i < dk; ++i) pred += kt[i] * S[(long)i * dv + j];
                u[j] = vh[(long)t * dv + j] - pred;
                if (pred_out) pred_out[(h * (long)T + t) * dv + j] = pred;
            }
            /* write: S += beta_t k_t u^T */
            for (int i = 0; i < dk; ++i) {
                const double bk = bh[t] * kt[i];
                for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += bk * u[j];
            }
            /* read: o_t = S_t^T q_t */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += qh[(long)t * dk + i] * S[(long)i * dv + j];
                oh[(long)t * dv + j] = acc;
            }
        }
        if (S_out) memcpy(S_out + h * (long)dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S); free(u);
    }
}

/* The plain delta rule (no gate). */
void delta_ref_forward(const double* q, const double* k, const double* v,
                       const double* beta, const double* S0,
                       double* o, double* S_out,
                       int B, int H, int T, int dk, int dv) {
    delta_gated_forward(q, k, v, beta, NULL, S0, o, S_out, NULL, B, H, T, dk, dv);
}

/* The gated delta rule: alpha [B][H][T], the per-token forgetting factor. */
void gated_delta_ref_forward(const double* q, const double* k, const double* v,
                             const double* beta, const double* alpha, const double* S0,
                             double* o, double* S_out,
                             int B, int H, int T, int dk, int dv) {
    delta_gated_forward(q, k, v, beta, alpha, S0, o, S_out, NULL, B, H, T, dk, dv);
}

/* Either rule (alpha NULL = ungated) with the optional prediction output. */
void delta_ref_forward_ex(const double* q, const double* k, const double* v,
                          const double* beta, const double* alpha, const double* S0,
                          double* o, double* S_out, double* pred,
                          int B, int H, int T, int dk, int dv) {
    delta_gated_forward(q, k, v, beta, alpha, S0, o, S_out, pred, B, H, T, dk, dv);
}

/*
 * One decode step of normalized linear attention on a resident state,
 * updated in place: S += phi(k) v^T, z += phi(k), then
 * o = phi(q)^T S / (phi(q)^T z + eps).  [LinearMem] §03 (the recurrence and
 * read-out) and §05 (inference keeps the matrix and normaliser state and
 * updates it in place, one token at a time).
 *   q, k [N][H][dk]   v, o [N][H][dv]   S [N][H][dk][dv]   z [N][H][dk]
 */
void la_ref_decode_step(const double* q, const double* k, const double* v,
                        double* S, double* z, double* o,
                        int N, int H, int dk, int dv, double eps) {
    const long states = (long)N * H;
#pragma omp parallel for schedule(static)
    for (long s = 0; s < states; ++s) {
        const double* qs = q + s * dk;
        const double* ks = k + s * dk;
        const double* vs = v + s * dv;
        double* Ss = S + s * (long)dk * dv;
        double* zs = z + s * dk;
        double den = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double f = phi_elu1(ks[i]);
            for (int j = 0; j < dv; ++j) Ss[(long)i * dv + j] += f * vs[j];
            zs[i] += f;
        }
        for (int i = 0; i < dk; ++i) den += phi_elu1(qs[i]) * zs[i];
        den += eps;
        for (int j = 0; j < dv; ++j) {
            double num = 0.0;
            for (int i = 0; i < dk; ++i) num += phi_elu1(qs[i]) * Ss[(long)i * dv + j];
            o[s * dv + j] = num / den;
        }
    }
}

/*
 * One decode step of the delta-rule fast-weight memory on a resident state,
 * updated in place ([LinearMem] §03 "从累加改成纠错" and [Recurrence]
 * "Delta-rule fast weight" for the write; §05 for updating the inference
 * state in place): the correction u = v - S^T k (the new value minus what the
 * memory predicts for k), then S += beta k u^T, then the write-then-read
 * output o = S^T q with the updated state.
 *   q, k [N][H][dk]   v, o [N][H][dv]   beta [N][H]   S [N][H][dk][dv]
 */
static void delta_gated_decode_step(const double* q, const double* k, const double* v,
                                    const double* beta, const double* alpha, double* S, double* o,
                                    double* pred_out, int N, int H, int dk, int dv) {
    const long states = (long)N * H;
#pragma omp parallel for schedule(static)
    for (long s = 0; s < states; ++s) {
        const double* qs = q + s * dk;
        const double* ks = k + s * dk;
        const double* vs = v + s * dv;
        double* Ss = S + s * (long)dk * dv;
        if (alpha)  /* forget first */
            for (long i = 0; i < (long)dk * dv; ++i) Ss[i] *= alpha[s];
        for (int j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (int i = 0; i < dk; ++i) pred += ks[i] * Ss[(long)i * dv + j];
            if (pred_out) pred_out[s * dv + j] = pred;
            const double u = vs[j] - pred;
            for (int i = 0; i < dk; ++i) Ss[(long)i * dv + j] += beta[s] * ks[i] * u;
        }
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += qs[i] * Ss[(long)i * dv + j];
            o[s * dv + j] = acc;
        }
    }
}

void delta_ref_decode_step(const double* q, const double* k, const double* v,
                           const double* beta, double* S, double* o,
                           int N, int H, int dk, int dv) {
    delta_gated_decode_step(q, k, v, beta, NULL, S, o, NULL, N, H, dk, dv);
}

/* The gated form of the step above: S is first scaled by alpha [N][H]. */
void gated_delta_ref_decode_step(const double* q, const double* k, const double* v,
                                 const double* beta, const double* alpha, double* S, double* o,
                                 int N, int H, int dk, int dv) {
    delta_gated_decode_step(q, k, v, beta, alpha, S, o, NULL, N, H, dk, dv);
}

/* Either step (alpha NULL = ungated) with the optional prediction output [N][H][dv]. */
void delta_ref_decode_step_ex(const double* q, const double* k, const double* v,
                              const double* beta, const double* alpha, double* S, double* o,
                              double* pred, int N, int H, int dk, int dv) {
    delta_gated_decode_step(q, k, v, beta, alpha, S, o, pred, N, H, dk, dv);
}

/*
 * Input transforms that a serving stack applies before the rule
 * ([LinearMem] §05: FLA hands the q/k L2 normalisation and the beta
 * transform to the kernel; §08: the model predicts a raw gate, and the
 * kernel applies a sigmoid to it):
 *   l2 rows:  y = x / ||x||_2 per row of d (a zero row stays zero);
 *   sigmoid:  y = 1 / (1 + e^-x).
 */
void oracle_l2_normalize_rows(const double* x, double* y, long rows, int d) {
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int i = 0; i < d; ++i) ss += x[r * d + i] * x[r * d + i];
        const double n = sqrt(ss);
        for (int i = 0; i < d; ++i) y[r * d + i] = n > 0.0 ? x[r * d + i] / n : 0.0;
    }
}

void oracle_sigmoid(const double* x, double* y, long n) {
    for (long i = 0; i < n; ++i) y[i] = 1.0 / (1.0 + exp(-x[i]));
}

/*
 * Scalar-decay linear memory, the Mamba-2 / SSD form ([LA-SSM] §3 "Mamba 一族",
 * Mamba-2 paragraph: the outer-product state with a scalar decay alpha_t on
 * the old state; written key-first here):
 *   S_t = alpha_t S_{t-1} + k_t v_t^T,    o_t = S_t^T q_t    (write, then read).
 * No feature map, no normaliser, no correction.  With d_k = d_v = 1 this is
 * the elementwise recurrence of [Recurrence] "Selective scan" with a = alpha,
 * b = k, x = v, c = q.  alpha [B][H][T].
 */
void ssd_ref_forward(const double* q, const double* k, const double* v, const double* alpha,
                     const double* S0, double* o, double* S_out,
                     int B, int H, int T, int dk, int dv) {
    const long heads = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < heads; ++h) {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        for (long i = 0; i < (long)dk * dv; ++i) S[i] = S0 ? S0[h * dk * dv + i] : 0.0;
        const double* qh = q + h * (long)T * dk;
        const double* kh = k + h * (long)T * dk;
        const double* vh = v + h * (long)T * dv;
        const double* ah = alpha + h * (long)T;
        double* oh = o + h * (long)T * dv;
        for (int t = 0; t < T; ++t) {
            const double* kt = kh + (long)t * dk;
            const double* vt = vh + (long)t * dv;
            const double* qt = qh + (long)t * dk;
            /* decay the old state, then add the outer product */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(long)i * dv + j] = ah[t] * S[(long)i * dv + j] + kt[i] * vt[j];
            /* read with the updated state */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += qt[i] * S[(long)i * dv + j];
                oh[(long)t * dv + j] = acc;
            }
        }
        if (S_out) memcpy(S_out + h * (long)dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
    }
}

/* One step of the rule above on a resident state S [N][H][dk][dv], in place;
 * alpha [N][H]. */
void ssd_ref_decode_step(const double* q, const double* k, const double* v, const double* alpha,
                         double* S, double* o, int N, int H, int dk, int dv) {
    const long states = (long)N * H;
#pragma omp parallel for schedule(static)
    for (long s = 0; s < states; ++s) {
        double* Ss = S + s * (long)dk * dv;
        const double* ks = k + s * (long)dk;
        const double* vs = v + s * (long)dv;
        const double* qs = q + s * (long)dk;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Ss[(long)i * dv + j] = alpha[s] * Ss[(long)i * dv + j] + ks[i] * vs[j];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += qs[i] * Ss[(long)i * dv + j];
            o[s * (long)dv + j] = acc;
        }
    }
}

/*
 * Backward pass of la_ref_forward (reverse-mode differentiation of the same
 * token recurrence).  [LinearMem] §03: storing every step's state makes
 * training memory grow with the length; prefix sums, chunking and
 * recomputation in the backward pass are the remedy.  This reference keeps
 * only per-token scalars: a forward sweep recomputes S_t, z_t and gives the
 * query gradients and d num_t, d den_t; a reverse sweep accumulates
 *   G_S = dS_T + sum_{s >= t} phi(q_s) dnum_s^T,  G_z = dz_T + sum_{s >= t} phi(q_s) dden_s
 * and gives the key and value gradients.  With the loss
 *   L = sum_t dO_t . o_t + <dS_T, S_T> + <dz_T, z_T>:
 *   dnum_t = dO_t / den_t,  dden_t = -(dO_t . num_t) / den_t^2   (normalize = 0: dnum = dO, dden = 0)
 *   dphi(q_t) = S_t dnum_t + z_t dden_t
 *   dphi(k_t) = G_S(t) v_t + G_z(t),  dv_t = G_S(t)^T phi(k_t)
 *   dS_0 = G_S(0), dz_0 = G_z(0); d u = dphi(u) phi'(u), phi'(u) = 1 (u > 0), e^u (u <= 0).
 * dS_T, dz_T may be NULL (zero); dS0, dz0 may be NULL (not returned).
 */
static double feature_grad(double u, int mode) {
    return mode == ORACLE_PHI_IDENTITY ? 1.0 : (u > 0.0 ? 1.0 : exp(u));
}

void la_ref_backward(const double* q, const double* k, const double* v, const double* S0, const double* z0,
                     const double* dO, const double* dS_T, const double* dz_T,
                     double* dq, double* dk_out, double* dv_out, double* dS0, double* dz0,
                     int B, int H, int T, int dk, int dv, double eps, int feature_mode, int normalize) {
    const long heads = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < heads; ++h) {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* z = (double*)malloc(sizeof(double) * (size_t)dk);
        double* fq = (double*)malloc(sizeof(double) * (size_t)dk);
        double* fk = (double*)malloc(sizeof(double) * (size_t)dk);
        double* num = (double*)malloc(sizeof(double) * (size_t)dv);
        double* dnum = (double*)malloc(sizeof(double) * (size_t)T * dv);
        double* dden = (double*)malloc(sizeof(double) * (size_t)T);
        const double* qh = q + h * (long)T * dk;
        const double* kh = k + h * (long)T * dk;
        const double* vh = v + h * (long)T * dv;
        const double* gh = dO + h * (long)T * dv;
        for (long i = 0; i < (long)dk * dv; ++i) S[i] = S0 ? S0[h * dk * dv + i] : 0.0;
        for (int i = 0; i < dk; ++i) z[i] = z0 ? z0[h * dk + i] : 0.0;
        /* forward sweep: states, d num, d den and the query gradients */
        for (int t = 0; t < T; ++t) {
            for (int i = 0; i < dk; ++i) {
                fk[i] = feature(kh[(long)t * dk + i], feature_mode);
                fq[i] = feature(qh[(long)t * dk + i], feature_mode);
            }
            for (int i = 0; i < dk; ++i) {
                for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += fk[i] * vh[(long)t * dv + j];
                z[i] += fk[i];
            }
            double den = eps;
            for (int i = 0; i < dk; ++i) den += fq[i] * z[i];
            double dot = 0.0;
            for (int j = 0; j < dv; ++j) {
                double a = 0.0;
                for (int i = 0; i < dk; ++i) a += fq[i] * S[(long)i * dv + j];
                num[j] = a;
                dot += gh[(long)t * dv + j] * a;
            }
            for (int j = 0; j < dv; ++j)
                dnum[(long)t * dv + j] = normalize ? gh[(long)t * dv + j] / den : gh[(long)t * dv + j];
            dden[t] = normalize ? -dot / (den * den) : 0.0;
            for (int i = 0; i < dk; ++i) {
                double a = z[i] * dden[t];
                for (int j = 0; j < dv; ++j) a += S[(long)i * dv + j] * dnum[(long)t * dv + j];
                dq[(h * (long)T + t) * dk + i] = a * feature_grad(qh[(long)t * dk + i], feature_mode);
            }
        }
        /* reverse sweep: G_S, G_z and the key and value gradients */
        for (long i = 0; i < (long)dk * dv; ++i) S[i] = dS_T ? dS_T[h * dk * dv + i] : 0.0;  /* G_S */
        for (int i = 0; i < dk; ++i) z[i] = dz_T ? dz_T[h * dk + i] : 0.0;                     /* G_z */
        for (int t = T - 1; t >= 0; --t) {
            for (int i = 0; i < dk; ++i) {
                fq[i] = feature(qh[(long)t * dk + i], feature_mode);
                fk[i] = feature(kh[(long)t * dk + i], feature_mode);
            }
            for (int i = 0; i < dk; ++i) {
                for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += fq[i] * dnum[(long)t * dv + j];
                z[i] += fq[i] * dden[t];
            }
            for (int i = 0; i < dk; ++i) {
                double a = z[i];
                for (int j = 0; j < dv; ++j) a += S[(long)i * dv + j] * vh[(long)t * dv + j];
                dk_out[(h * (long)T + t) * dk + i] = a * feature_grad(kh[(long)t * dk + i], feature_mode);
            }
            for (int j = 0; j < dv; ++j) {
                double a = 0.0;
                for (int i = 0; i < dk; ++i) a += S[(long)i * dv + j] * fk[i];
                dv_out[(h * (long)T + t) * dv + j] = a;
            }
        }
        if (dS0) memcpy(dS0 + h * (long)dk * dv, S, sizeof(double) * (size_t)dk * dv);
        if (dz0) memcpy(dz0 + h * (long)dk, z, sizeof(double) * (size_t)dk);
        free(S); free(z); free(fq); free(fk); free(num); free(dnum); free(dden);
    }
}

/*
 * Backward pass of the (optionally gated) delta rule, reverse-mode
 * differentiation of the token recurrence of delta_gated_forward:
 *   S~ = alpha_t S_{t-1},  u_t = v_t - S~^T k_t,  S_t = S~ + beta_t k_t u_t^T,  o_t = S_t^T q_t,
 * for the loss L = sum_t dO_t . o_t + <dS_T, S_T>.  With G = dL/dS_t (running,
 * from dS_T):
 *   G += q_t dO_t^T,  dq_t = S_t dO_t,
 *   dbeta_t = k_t^T G u_t,  du_t = beta_t G^T k_t,  dv_t = du_t,
 *   dk_t = beta_t G u_t - S~ du_t,
 *   dS~ = G - k_t du_t^T,  dalpha_t = <dS~, S_{t-1}>,  G <- alpha_t dS~.
 * dS_0 = G at the end.  States are recomputed from checkpoints kept every 64
 * tokens (the [LinearMem] §03 remedy for training memory), so the memory is
 * O(T/64 dk dv + 64 dk dv) per head.  alpha NULL: the plain rule (dalpha not
 * written); dS_T, dS0 and dalpha may be NULL.
 */
void delta_ref_backward(const double* q, const double* k, const double* v, const double* beta,
                        const double* alpha, const double* S0, const double* dO, const double* dS_T,
                        double* dq, double* dk_out, double* dv_out, double* dbeta, double* dalpha, double* dS0,
                        int B, int H, int T, int dk, int dv) {
    const long heads = (long)B * H;
    const int CK = 64;
    const int nck = (T + CK - 1) / CK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < heads; ++h) {
        const long E = (long)dk * dv;
        double* ck = (double*)malloc(sizeof(double) * (size_t)nck * E);        /* state entering each block */
        double* blk = (double*)malloc(sizeof(double) * (size_t)(CK + 1) * E);  /* states of one block */
        double* us = (double*)malloc(sizeof(double) * (size_t)CK * dv);        /* its corrections */
        double* G = (double*)malloc(sizeof(double) * (size_t)E);
        double* dSt = (double*)malloc(sizeof(double) * (size_t)E);
        double* du = (double*)malloc(sizeof(double) * (size_t)dv);
        const double* qh = q + h * (long)T * dk;
        const double* kh = k + h * (long)T * dk;
        const double* vh = v + h * (long)T * dv;
        const double* bh = beta + h * (long)T;
        const double* ah = alpha ? alpha + h * (long)T : NULL;
        const double* gh = dO + h * (long)T * dv;
        /* forward sweep: checkpoints only */
        for (long i = 0; i < E; ++i) blk[i] = S0 ? S0[h * E + i] : 0.0;
        for (int t = 0; t < T; ++t) {
            if (t % CK == 0) memcpy(ck + (long)(t / CK) * E, blk, sizeof(double) * (size_t)E);
            const double* kt = kh + (long)t * dk;
            if (ah) for (long i = 0; i < E; ++i) blk[i] *= ah[t];
            for (int j = 0; j < dv; ++j) {
                double p = 0.0;
                for (int i = 0; i < dk; ++i) p += kt[i] * blk[(long)i * dv + j];
                du[j] = vh[(long)t * dv + j] - p;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) blk[(long)i * dv + j] += bh[t] * kt[i] * du[j];
        }
        /* reverse sweep, block by block */
        for (long i = 0; i < E; ++i) G[i] = dS_T ? dS_T[h * E + i] : 0.0;
        for (int b = nck - 1; b >= 0; --b) {
            const int t0 = b * CK, n = (T - t0) < CK ? (T - t0) : CK;
            /* recompute the block: blk[s] = state before token t0 + s, us[s] = its correction */
            memcpy(blk, ck + (long)b * E, sizeof(double) * (size_t)E);
            for (int s2 = 0; s2 < n; ++s2) {
                const int t = t0 + s2;
                const double* kt = kh + (long)t * dk;
                double* cur = blk + (long)s2 * E;
                double* nxt = blk + (long)(s2 + 1) * E;
                const double a = ah ? ah[t] : 1.0;
                for (int j = 0; j < dv; ++j) {
                    double p = 0.0;
                    for (int i = 0; i < dk; ++i) p += kt[i] * a * cur[(long)i * dv + j];
                    us[(long)s2 * dv + j] = vh[(long)t * dv + j] - p;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        nxt[(long)i * dv + j] = a * cur[(long)i * dv + j] + bh[t] * kt[i] * us[(long)s2 * dv + j];
            }
            for (int s2 = n - 1; s2 >= 0; --s2) {
                const int t = t0 + s2;
                const double* kt = kh + (long)t * dk;
                const double* qt = qh + (long)t * dk;
                const double* prev = blk + (long)s2 * E;   /* S_{t-1} */
                const double* post = blk + (long)(s2 + 1) * E;  /* S_t */
                const double* ut = us + (long)s2 * dv;
                const double a = ah ? ah[t] : 1.0;
                /* the read o_t = S_t^T q_t */
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        acc += post[(long)i * dv + j] * gh[(long)t * dv + j];
                        G[(long)i * dv + j] += qt[i] * gh[(long)t * dv + j];
                    }
                    dq[(h * (long)T + t) * dk + i] = acc;
                }
                /* the write S_t = S~ + beta_t k_t u_t^T */
                double db = 0.0;
                for (int j = 0; j < dv; ++j) {
                    double gk = 0.0;
                    for (int i = 0; i < dk; ++i) gk += G[(long)i * dv + j] * kt[i];
                    db += gk * ut[j];
                    du[j] = bh[t] * gk;
                    dv_out[(h * (long)T + t) * dv + j] = du[j];
                }
                dbeta[h * (long)T + t] = db;
                for (int i = 0; i < dk; ++i) {
                    double gu = 0.0, sd = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        gu += G[(long)i * dv + j] * ut[j];
                        sd += a * prev[(long)i * dv + j] * du[j];
                    }
                    dk_out[(h * (long)T + t) * dk + i] = bh[t] * gu - sd;
                }
                /* dS~ = G - k_t du^T, then through S~ = alpha_t S_{t-1} */
                double dal = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) {
                        const double x = G[(long)i * dv + j] - kt[i] * du[j];
                        dSt[(long)i * dv + j] = x;
                        dal += x * prev[(long)i * dv + j];
                    }
                if (dalpha && ah) dalpha[h * (long)T + t] = dal;
                for (long i = 0; i < E; ++i) G[i] = a * dSt[i];
            }
        }
        if (dS0) memcpy(dS0 + h * E, G, sizeof(double) * (size_t)E);
        free(ck); free(blk); free(us); free(G); free(dSt); free(du);
    }
}

/* The feature map alone, so tests can pin its branches directly. */
void oracle_phi(const double* x, double* y, long n) {
    for (long i = 0; i < n; ++i) y[i] = phi_elu1(x[i]);
}

/* Threads OpenMP will use for the loops above (1 when built without it). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
