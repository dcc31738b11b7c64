/*
 * attn_oracle.c -- plain, slow, obviously correct CPU reference for causal
 * grouped-query attention, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * What it computes is the plain definition of softmax attention, written out
 * step by step with the score and probability matrices of one head fully
 * materialised.  The method on the pages ("tang -- differentiable computing in
 * Rust", section "How tang works", part 3 "Optimizations are derived, not
 * written", equations (5) and (6)) reaches exactly this result up to rounding
 * order: it rewrites the max and the two sums of the softmax into one
 * streaming reduction, but the value it computes is unchanged.  The equations
 * themselves did not survive text extraction; the reading used here is the
 * textbook max-subtracted softmax for (5) and the (max, sum, weighted sum)
 * running state for (6), the only reading consistent with the surrounding
 * prose ("the max and the two sums", "three running values").
 *
 * Conventions (the pages are silent on these; readings stated here):
 *   - layouts are contiguous row-major with the head dimension fastest:
 *       q, o, dout, dq : [B][Hq][Nq][d]     k, v, dk, dv : [B][Hkv][Nk][d]
 *       lse            : [B][Hq][Nq]
 *   - grouped-query head map: query head h reads key/value head h / (Hq/Hkv)
 *     (contiguous groups); Hq must be a multiple of Hkv.
 *   - causal visibility: key j is visible to query i iff j <= i + (Nk - Nq)
 *     (bottom-right alignment; j <= i when Nq == Nk).
 *   - lse is the natural logarithm of the row's softmax denominator in
 *     absolute terms: lse_i = m_i + ln(l_i).
 *   - a row with no visible key gets o = 0 and lse = -inf.
 *
 * Parity status of each function is stated beside it; every function is
 * pinned by CPU tests against closed forms, invariants, finite differences,
 * dual numbers or an independent textbook computation.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NOMEM 2

static int is_visible(int causal, long i, long j, long Nq, long Nk)
{
    return !causal || j <= i + (Nk - Nq);
}

static int bad_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d)
{
    return B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || Hq % Hkv != 0;
}

/* ------------------------------------------------------------------------ */
/* Forward.                                                                  */
/* Steps, for one (b, h) with g = h / (Hq/Hkv):                              */
/*   1. s_ij = scale * <q_i, k_j>                                            */
/*   2. visibility mask                                                      */
/*   3. m_i = max over visible j of s_ij                                     */
/*   4. e_ij = exp(s_ij - m_i) (0 if masked)                                 */
/*   5. l_i  = sum_j e_ij                                                    */
/*   6. P_ij = e_ij / l_i        (materialised)                              */
/*   7. o_i  = sum_j P_ij v_j                                                */
/*   8. lse_i = m_i + ln l_i                                                 */
/* Source: the textbook softmax that the "How tang works" part 3 rewrite     */
/* starts from (equation (5)), applied per query head with the GQA sharing   */
/* of "RustingBrain" docs, "What is in the box" (grouped-query attention)    */
/* and the causal mask of its fused causal flash-attention kernel.           */
/* ------------------------------------------------------------------------ */

/* Fills P (Nq x Nk, row-major) for one head and writes lse for that head. */
static void head_probs(long Nq, long Nk, int d, int causal, double scale,
                       const double *qh, const double *kg, double *P, double *lse_h)
{
    long i;
#pragma omp parallel for schedule(dynamic, 4)
    for (i = 0; i < Nq; ++i) {
        double *Pi = P + i * Nk;
        double m = -INFINITY;
        long j;
        int c;
        for (j = 0; j < Nk; ++j) {
            if (!is_visible(causal, i, j, Nq, Nk)) { Pi[j] = -INFINITY; continue; }
            double s = 0.0;
            for (c = 0; c < d; ++c) s += qh[i * d + c] * kg[j * d + c];
            s *= scale;                                     /* step 1 */
            Pi[j] = s;
            if (s > m) m = s;                               /* step 3 */
        }
        if (m == -INFINITY) {                               /* no visible key */
            for (j = 0; j < Nk; ++j) Pi[j] = 0.0;
            lse_h[i] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (j = 0; j < Nk; ++j) {
            double e = (Pi[j] == -INFINITY) ? 0.0 : exp(Pi[j] - m);  /* step 4 */
            Pi[j] = e;
            l += e;                                         /* step 5 */
        }
        for (j = 0; j < Nk; ++j) Pi[j] /= l;                /* step 6 */
        lse_h[i] = m + log(l);                              /* step 8 */
    }
}

/* o_h = P v_g  (step 7) */
static void head_out(long Nq, long Nk, int d, const double *P, const double *vg, double *oh)
{
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < Nq; ++i) {
        int c;
        long j;
        for (c = 0; c < d; ++c) oh[i * d + c] = 0.0;
        for (j = 0; j < Nk; ++j) {
            double p = P[i * Nk + j];
            if (p == 0.0) continue;
            for (c = 0; c < d; ++c) oh[i * d + c] += p * vg[j * d + c];
        }
    }
}

/* Parity: pinned (closed forms, numpy textbook softmax, invariants). */
int oracle_attn_fwd(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, double scale,
                    const double *q, const double *k, const double *v,
                    double *o, double *lse)
{
    if (bad_shape(B, Hq, Hkv, Nq, Nk, d)) return ORACLE_BAD_ARG;
    int G = Hq / Hkv;
    double *P = (double *)malloc(sizeof(double) * (size_t)Nq * (size_t)Nk);
    if (!P) return ORACLE_NOMEM;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            const double *qh = q + ((size_t)b * Hq + h) * (size_t)Nq * d;
            const double *kg = k + ((size_t)b * Hkv + g) * (size_t)Nk * d;
            const double *vg = v + ((size_t)b * Hkv + g) * (size_t)Nk * d;
            double *oh = o + ((size_t)b * Hq + h) * (size_t)Nq * d;
            double *lh = lse + ((size_t)b * Hq + h) * (size_t)Nq;
            head_probs(Nq, Nk, d, causal, scale, qh, kg, P, lh);
            head_out(Nq, Nk, d, P, vg, oh);
        }
    free(P);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward, the analytic gradient of the forward for an upstream dO and an  */
/* upstream gradient dlse of lse (oracle_attn_bwd: dlse = 0):                */
/*    9. D_i   = <dO_i, o_i>                                                 */
/*   10. dP_ij = <dO_i, v_j>                                                 */
/*   11. dS_ij = P_ij (dP_ij - D_i + dlse_i)   (d lse_i / d s_ij = P_ij)     */
/*   12. dq_i  = scale * sum_j dS_ij k_j                                     */
/*   13. dk_j  = scale * sum_{h in group} sum_i dS_ij q_i                    */
/*   14. dv_j  = sum_{h in group} sum_i P_ij dO_i                            */
/* Source: the gradient of the same comprehension ("How tang works" part 3: */
/* gradients are comprehensions too; the compiler-article paragraph on views */
/* and comprehensions).  Written out from the chain rule through softmax.    */
/* Parity: pinned (central finite differences, dual numbers, invariants).    */
/* ------------------------------------------------------------------------ */
static int attn_bwd_impl(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, double scale,
                         const double *q, const double *k, const double *v, const double *dout,
                         const double *dlse, double *dq, double *dk, double *dv)
{
    if (bad_shape(B, Hq, Hkv, Nq, Nk, d)) return ORACLE_BAD_ARG;
    int G = Hq / Hkv;
    size_t NN = (size_t)Nq * (size_t)Nk;
    double *P = (double *)malloc(sizeof(double) * NN);
    double *dS = (double *)malloc(sizeof(double) * NN);
    double *oh = (double *)malloc(sizeof(double) * (size_t)Nq * d);
    double *lh = (double *)malloc(sizeof(double) * (size_t)Nq);
    double *Dv = (double *)malloc(sizeof(double) * (size_t)Nq);
    if (!P || !dS || !oh || !lh || !Dv) {
        free(P); free(dS); free(oh); free(lh); free(Dv);
        return ORACLE_NOMEM;
    }
    memset(dk, 0, sizeof(double) * (size_t)B * Hkv * Nk * d);
    memset(dv, 0, sizeof(double) * (size_t)B * Hkv * Nk * d);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            const double *qh = q + ((size_t)b * Hq + h) * (size_t)Nq * d;
            const double *doh = dout + ((size_t)b * Hq + h) * (size_t)Nq * d;
            const double *kg = k + ((size_t)b * Hkv + g) * (size_t)Nk * d;
            const double *vg = v + ((size_t)b * Hkv + g) * (size_t)Nk * d;
            double *dqh = dq + ((size_t)b * Hq + h) * (size_t)Nq * d;
            double *dkg = dk + ((size_t)b * Hkv + g) * (size_t)Nk * d;
            double *dvg = dv + ((size_t)b * Hkv + g) * (size_t)Nk * d;
            const double *dlh = dlse ? dlse + ((size_t)b * Hq + h) * (size_t)Nq : NULL;
            long i, j;

            head_probs(Nq, Nk, d, causal, scale, qh, kg, P, lh);
            head_out(Nq, Nk, d, P, vg, oh);

#pragma omp parallel for schedule(dynamic, 4)
            for (i = 0; i < Nq; ++i) {
                int c;
                double Di = 0.0;
                for (c = 0; c < d; ++c) Di += doh[i * d + c] * oh[i * d + c];   /* step 9 */
                Dv[i] = Di;
                double gl = dlh ? dlh[i] : 0.0;
                for (j = 0; j < Nk; ++j) {
                    double p = P[i * Nk + j];
                    if (p == 0.0) { dS[i * Nk + j] = 0.0; continue; }
                    double dp = 0.0;
                    for (c = 0; c < d; ++c) dp += doh[i * d + c] * vg[j * d + c]; /* step 10 */
                    dS[i * Nk + j] = p * (dp - Di + gl);                         /* step 11 */
                }
                for (c = 0; c < d; ++c) dqh[i * d + c] = 0.0;
                for (j = 0; j < Nk; ++j) {
                    double s = dS[i * Nk + j];
                    if (s == 0.0) continue;
                    for (c = 0; c < d; ++c) dqh[i * d + c] += s * kg[j * d + c];
                }
                for (c = 0; c < d; ++c) dqh[i * d + c] *= scale;                   /* step 12 */
            }
#pragma omp parallel for schedule(dynamic, 4)
            for (j = 0; j < Nk; ++j) {
                int c;
                for (i = 0; i < Nq; ++i) {
                    double s = dS[i * Nk + j], p = P[i * Nk + j];
                    if (p == 0.0 && s == 0.0) continue;                          /* masked */
                    for (c = 0; c < d; ++c) {
                        dkg[j * d + c] += scale * s * qh[i * d + c];              /* step 13 */
                        dvg[j * d + c] += p * doh[i * d + c];                      /* step 14 */
                    }
                }
            }
        }
    free(P); free(dS); free(oh); free(lh); free(Dv);
    return ORACLE_OK;
}

int oracle_attn_bwd(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, double scale,
                    const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv)
{
    return attn_bwd_impl(B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, dout, NULL, dq, dk, dv);
}

/* Backward with an upstream gradient dlse [B][Hq][Nq] of lse as well.        */
/* Parity: pinned (central finite differences of <o, dO> + <lse, dlse>, and  */
/* the dual-number directional derivative of o and lse).                     */
int oracle_attn_bwd_dlse(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, double scale,
                         const double *q, const double *k, const double *v, const double *dout,
                         const double *dlse, double *dq, double *dk, double *dv)
{
    return attn_bwd_impl(B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, dout, dlse, dq, dk, dv);
}

/* ------------------------------------------------------------------------ */
/* Dual numbers (forward-mode differentiation), used only to pin the         */
/* backward above.  A dual number carries a value and an infinitesimal part  */
/* e with e*e = 0, so any function evaluated on it returns its value and its */
/* exact directional derivative together ("tang -- differentiable computing  */
/* in Rust", "How tang works" part 1 "Dual numbers carry the derivative",    */
/* equations (1) and (2); the running example there is f(x) = x sin x).      */
/* Parity: pinned (f(x) = x sin x against its derivative sin x + x cos x,    */
/* including the page's printed x = 0 state).                                 */
/* ------------------------------------------------------------------------ */
typedef struct { double v, e; } dual;

static dual dl_make(double v, double e) { dual r; r.v = v; r.e = e; return r; }
static dual dl_add(dual a, dual b) { return dl_make(a.v + b.v, a.e + b.e); }
static dual dl_sub(dual a, dual b) { return dl_make(a.v - b.v, a.e - b.e); }
static dual dl_mul(dual a, dual b) { return dl_make(a.v * b.v, a.v * b.e + a.e * b.v); }
static dual dl_div(dual a, dual b)
{
    return dl_make(a.v / b.v, (a.e * b.v - a.v * b.e) / (b.v * b.v));
}
static dual dl_exp(dual a) { double x = exp(a.v); return dl_make(x, x * a.e); }
static dual dl_log(dual a) { return dl_make(log(a.v), a.e / a.v); }
static dual dl_sin(dual a) { return dl_make(sin(a.v), cos(a.v) * a.e); }

int oracle_dual_xsinx(double x, double *val, double *der)
{
    dual X = dl_make(x, 1.0);
    dual f = dl_mul(X, dl_sin(X));
    *val = f.v;
    *der = f.e;
    return ORACLE_OK;
}

/* The forward steps 1-8 evaluated on dual numbers: inputs (x, tx) give      */
/* outputs (o, to) and (lse, tlse), the tangents being the exact directional  */
/* derivatives of o and lse along (tq, tk, tv).                              */
int oracle_attn_fwd_dual(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, double scale,
                         const double *q, const double *tq, const double *k, const double *tk,
                         const double *v, const double *tv,
                         double *o, double *to, double *lse, double *tlse)
{
    if (bad_shape(B, Hq, Hkv, Nq, Nk, d)) return ORACLE_BAD_ARG;
    int G = Hq / Hkv;
    dual *S = (dual *)malloc(sizeof(dual) * (size_t)Nk);
    if (!S) return ORACLE_NOMEM;
    dual sc = dl_make(scale, 0.0);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            size_t qo = ((size_t)b * Hq + h) * (size_t)Nq * d;
            size_t ko = ((size_t)b * Hkv + g) * (size_t)Nk * d;
            size_t lo = ((size_t)b * Hq + h) * (size_t)Nq;
            for (long i = 0; i < Nq; ++i) {
                long jmax = -1;
                for (long j = 0; j < Nk; ++j) {
                    if (!is_visible(causal, i, j, Nq, Nk)) continue;
                    dual s = dl_make(0.0, 0.0);
                    for (int c = 0; c < d; ++c) {
                        dual qc = dl_make(q[qo + i * d + c], tq[qo + i * d + c]);
                        dual kc = dl_make(k[ko + j * d + c], tk[ko + j * d + c]);
                        s = dl_add(s, dl_mul(qc, kc));
                    }
                    S[j] = dl_mul(sc, s);
                    if (jmax < 0 || S[j].v > S[jmax].v) jmax = j;
                }
                if (jmax < 0) {
                    for (int c = 0; c < d; ++c) { o[qo + i * d + c] = 0.0; to[qo + i * d + c] = 0.0; }
                    lse[lo + i] = -INFINITY;
                    tlse[lo + i] = 0.0;
                    continue;
                }
                dual m = S[jmax];
                dual l = dl_make(0.0, 0.0);
                for (long j = 0; j < Nk; ++j) {
                    if (!is_visible(causal, i, j, Nq, Nk)) continue;
                    S[j] = dl_exp(dl_sub(S[j], m));
                    l = dl_add(l, S[j]);
                }
                for (int c = 0; c < d; ++c) {
                    dual acc = dl_make(0.0, 0.0);
                    for (long j = 0; j < Nk; ++j) {
                        if (!is_visible(causal, i, j, Nq, Nk)) continue;
                        dual vc = dl_make(v[ko + j * d + c], tv[ko + j * d + c]);
                        acc = dl_add(acc, dl_mul(dl_div(S[j], l), vc));
                    }
                    o[qo + i * d + c] = acc.v;
                    to[qo + i * d + c] = acc.e;
                }
                dual L = dl_add(m, dl_log(l));
                lse[lo + i] = L.v;
                tlse[lo + i] = L.e;
            }
        }
    free(S);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Split-KV decode.  One query token per (b, h) sits after all L cached keys, */
/* so every key is visible to it ("RustingBrain" docs, "Generating text":    */
/* after the prefill each token costs one row of attention against the      */
/* cache).  The L keys are cut into S contiguous chunks of C = ceil(L/S)     */
/* keys; chunk s covers [s*C, min((s+1)*C, L)).  Each chunk runs forward     */
/* steps 1-8 on its own keys and yields a partial (o_s, lse_s); an empty     */
/* chunk yields (0, -inf).                                                   */
/* q : [B][Hq][d]   k_cache, v_cache : [B][Hkv][L][d]                        */
/* part_o : [B][Hq][S][d]   part_lse : [B][Hq][S]                            */
/* Parity: pinned (the merged result equals the unsplit definition for any   */
/* S, and equals the last row of a causal forward).                          */
/* ------------------------------------------------------------------------ */
int oracle_attn_decode(int B, int Hq, int Hkv, int L, int d, double scale, int S,
                       const double *q, const double *kc, const double *vc,
                       double *part_o, double *part_lse)
{
    if (bad_shape(B, Hq, Hkv, 1, L, d) || S <= 0) return ORACLE_BAD_ARG;
    int G = Hq / Hkv;
    long C = ((long)L + S - 1) / S;
    double *e = (double *)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    if (!e) return ORACLE_NOMEM;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            const double *qh = q + ((size_t)b * Hq + h) * d;
            const double *kg = kc + ((size_t)b * Hkv + g) * (size_t)L * d;
            const double *vg = vc + ((size_t)b * Hkv + g) * (size_t)L * d;
            for (int s = 0; s < S; ++s) {
                double *po = part_o + (((size_t)b * Hq + h) * S + s) * d;
                double *pl = part_lse + ((size_t)b * Hq + h) * S + s;
                long j0 = (long)s * C, j1 = j0 + C;
                if (j1 > L) j1 = L;
                if (j0 >= j1) {
                    for (int c = 0; c < d; ++c) po[c] = 0.0;
                    *pl = -INFINITY;
                    continue;
                }
                double m = -INFINITY;
                for (long j = j0; j < j1; ++j) {
                    double sc = 0.0;
                    for (int c = 0; c < d; ++c) sc += qh[c] * kg[j * d + c];
                    sc *= scale;
                    e[j - j0] = sc;
                    if (sc > m) m = sc;
                }
                double l = 0.0;
                for (long j = j0; j < j1; ++j) {
                    e[j - j0] = exp(e[j - j0] - m);
                    l += e[j - j0];
                }
                for (int c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (long j = j0; j < j1; ++j) acc += (e[j - j0] / l) * vg[j * d + c];
                    po[c] = acc;
                }
                *pl = m + log(l);
            }
        }
    free(e);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Merge of split partials by their log-sum-exp.  The (max, sum, weighted    */
/* sum) state of the online softmax combines associatively ("How tang works" */
/* part 3: the combine is associative, so it tiles and parallelises like any */
/* sum).  In the normalised form (o_s, lse_s) the combine is                 */
/*   M = max_s lse_s,  w_s = exp(lse_s - M),                                 */
/*   o = sum_s w_s o_s / sum_s w_s,  lse = M + ln sum_s w_s.                 */
/* If every chunk is empty (M = -inf) the result is o = 0, lse = -inf.        */
/* Parity: pinned (order independence over permutations and merge trees,     */
/* identity and associativity, equality with the unsplit definition).        */
/* ------------------------------------------------------------------------ */
int oracle_lse_merge(int B, int Hq, int S, int d, const double *part_o, const double *part_lse,
                     double *o, double *lse)
{
    if (B <= 0 || Hq <= 0 || S <= 0 || d <= 0) return ORACLE_BAD_ARG;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            const double *po = part_o + ((size_t)b * Hq + h) * (size_t)S * d;
            const double *pl = part_lse + ((size_t)b * Hq + h) * S;
            double *oo = o + ((size_t)b * Hq + h) * d;
            double M = -INFINITY;
            for (int s = 0; s < S; ++s) if (pl[s] > M) M = pl[s];
            if (M == -INFINITY) {
                for (int c = 0; c < d; ++c) oo[c] = 0.0;
                lse[(size_t)b * Hq + h] = -INFINITY;
                continue;
            }
            double W = 0.0;
            for (int c = 0; c < d; ++c) oo[c] = 0.0;
            for (int s = 0; s < S; ++s) {
                if (pl[s] == -INFINITY) continue;
                double w = exp(pl[s] - M);
                W += w;
                for (int c = 0; c < d; ++c) oo[c] += w * po[(size_t)s * d + c];
            }
            for (int c = 0; c < d; ++c) oo[c] /= W;
            lse[(size_t)b * Hq + h] = M + log(W);
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* The online-softmax state and its combine, in un-normalised form: a state  */
/* (m, l, a) holds a running max m, the sum l of exp(s - m) and the weighted */
/* sum a of exp(s - m) v.  A key with score s and value v enters as          */
/* (s, 1, v); two states combine as                                          */
/*   m = max(m1, m2),  l = l1 e^(m1-m) + l2 e^(m2-m),                          */
/*   a = a1 e^(m1-m) + a2 e^(m2-m);                                           */
/* the identity is (-inf, 0, 0), applied as a rule.  The result of a fold is */
/* o = a / l, lse = m + ln l.  ("How tang works" part 3, equation (6): three  */
/* running values carried per query row while the keys stream past.)        */
/* Parity: pinned (folds in random orders and trees equal the materialised   */
/* softmax; identity and associativity laws).                               */
/* ------------------------------------------------------------------------ */
void oracle_state_combine(int d, double m1, double l1, const double *a1,
                          double m2, double l2, const double *a2,
                          double *m, double *l, double *a)
{
    if (m1 == -INFINITY) {                     /* identity on the left */
        *m = m2; *l = l2;
        for (int c = 0; c < d; ++c) a[c] = a2[c];
        return;
    }
    if (m2 == -INFINITY) {                     /* identity on the right */
        *m = m1; *l = l1;
        for (int c = 0; c < d; ++c) a[c] = a1[c];
        return;
    }
    double mm = m1 > m2 ? m1 : m2;
    double w1 = exp(m1 - mm), w2 = exp(m2 - mm);
    *l = l1 * w1 + l2 * w2;
    for (int c = 0; c < d; ++c) a[c] = a1[c] * w1 + a2[c] * w2;
    *m = mm;
}

/* ------------------------------------------------------------------------ */
/* One decode step against a growing cache ("RustingBrain" docs, "Generating */
/* text": after the prefill, each new token's key and value join the cache    */
/* and the token costs one row of attention over it).  For sequence b with   */
/* n = seq_lens[b] tokens already cached (0 <= n < Lcap):                    */
/*   1. append: the new token's key and value are written at cache row n of */
/*      every key/value head;                                                */
/*   2. each query head h (kv head g = h / (Hq/Hkv)) attends over the n + 1  */
/*      keys 0..n, all visible (the token sits after the cache):             */
/*      s_j = scale <q, k_j>, m = max s_j, l = sum exp(s_j - m),             */
/*      o = sum exp(s_j - m) v_j / l, lse = m + ln l.                        */
/* A length outside [0, Lcap) is reported, not clamped (reading; the pages   */
/* are silent): that sequence's cache is left untouched and its o and lse    */
/* are NaN.                                                                  */
/* q : [B][Hq][d]   k_new, v_new : [B][Hkv][d]   kc, vc : [B][Hkv][Lcap][d]  */
/* seq_lens : [B]   o : [B][Hq][d]   lse : [B][Hq]                           */
/* Parity: pinned (closed forms at n = 0 and for identical keys, equality    */
/* with the last row of a causal forward, the cache rows after the append,   */
/* rows past n without influence, invalid lengths).                          */
/* ------------------------------------------------------------------------ */
int oracle_attn_decode_append(int B, int Hq, int Hkv, int Lcap, int d, double scale,
                              const double *q, const double *k_new, const double *v_new,
                              double *kc, double *vc, const int *seq_lens, double *o,
                              double *lse)
{
    if (bad_shape(B, Hq, Hkv, 1, Lcap, d)) return ORACLE_BAD_ARG;
    int G = Hq / Hkv;
    double *e = (double *)malloc(sizeof(double) * (size_t)Lcap);
    if (!e) return ORACLE_NOMEM;
    for (int b = 0; b < B; ++b) {
        long n = seq_lens[b];
        if (n < 0 || n >= Lcap) {
            for (int h = 0; h < Hq; ++h) {
                for (int c = 0; c < d; ++c) o[((size_t)b * Hq + h) * d + c] = NAN;
                lse[(size_t)b * Hq + h] = NAN;
            }
            continue;
        }
        /* step 1: append */
        for (int g = 0; g < Hkv; ++g) {
            double *krow = kc + (((size_t)b * Hkv + g) * (size_t)Lcap + n) * d;
            double *vrow = vc + (((size_t)b * Hkv + g) * (size_t)Lcap + n) * d;
            for (int c = 0; c < d; ++c) {
                krow[c] = k_new[((size_t)b * Hkv + g) * d + c];
                vrow[c] = v_new[((size_t)b * Hkv + g) * d + c];
            }
        }
        /* step 2: one row of attention over keys 0..n */
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            const double *qh = q + ((size_t)b * Hq + h) * d;
            const double *kg = kc + ((size_t)b * Hkv + g) * (size_t)Lcap * d;
            const double *vg = vc + ((size_t)b * Hkv + g) * (size_t)Lcap * d;
            double m = -INFINITY;
            for (long j = 0; j <= n; ++j) {
                double sc = 0.0;
                for (int c = 0; c < d; ++c) sc += qh[c] * kg[j * d + c];
                e[j] = scale * sc;
                if (e[j] > m) m = e[j];
            }
            double l = 0.0;
            for (long j = 0; j <= n; ++j) {
                e[j] = exp(e[j] - m);
                l += e[j];
            }
            double *oh = o + ((size_t)b * Hq + h) * d;
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (long j = 0; j <= n; ++j) acc += e[j] * vg[j * d + c];
                oh[c] = acc / l;
            }
            lse[(size_t)b * Hq + h] = m + log(l);
        }
    }
    free(e);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Rotary positions.  The pages name rotary position embeddings beside GQA   */
/* attention among the derived ops ("tang -- differentiable computing in     */
/* Rust", the "A transformer" panel; RustingBrain docs, "What is in the      */
/* box") but print no formula.  Reading: the usual rotary embedding on       */
/* paired halves of the head dimension.  For a row at position p and pair   */
/* index i in [0, d/2):                                                      */
/*   theta_i = base^(-2i/d),  a = p * theta_i,                               */
/*   y_i       = x_i cos a - x_{i+d/2} sin a                                 */
/*   y_{i+d/2} = x_i sin a + x_{i+d/2} cos a                                 */
/* and with inverse != 0 the transposed rotation (angle -a), which is also   */
/* the map that carries a gradient with respect to y back to x.  Row n of    */
/* each [N][d] head sits at position pos0 + n.                               */
/* Parity: pinned (identity at p = 0, pair norms kept, scores depend only on */
/* the position difference, a d = 2 closed form, inverse after forward is    */
/* the identity, finite differences through attention).                      */
/* ------------------------------------------------------------------------ */
int oracle_rope(int B, int H, int N, int d, long pos0, double base, int inverse,
                const double *x, double *y)
{
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || d % 2 != 0 || !(base > 0.0)) return ORACLE_BAD_ARG;
    int half = d / 2;
    double sgn = inverse ? -1.0 : 1.0;
    for (long r = 0; r < (long)B * H * N; ++r) {
        long p = pos0 + r % N;
        const double *xr = x + r * d;
        double *yr = y + r * d;
        for (int i = 0; i < half; ++i) {
            double theta = pow(base, -2.0 * i / d);
            double a = (double)p * theta;
            double c = cos(a), s = sgn * sin(a);
            double x0 = xr[i], x1 = xr[i + half];
            yr[i] = x0 * c - x1 * s;
            yr[i + half] = x0 * s + x1 * c;
        }
    }
    return ORACLE_OK;
}

int oracle_abi_version(void) { return 1; }

/* Number of host threads the parallel loops above use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
