/*
 * fp64 CPU oracle for the Gated DeltaNet forward and its span summary.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code with the GPU library.
 *
 * What it computes (plain definition, token by token, no chunking):
 *
 *   The cuDNN "Linear Attention" page (opening paragraph) describes a recurrent
 *   matrix state S per (sequence, head); its "Semantics worth knowing" list
 *   ("Summaries") calls the span operator the product of the span's decayed
 *   erase steps, and the cudnn-frontend PR "Further reduce FROST LA CPU
 *   overhead + fully support all L2norm, beta, gate fusion" states that the
 *   gate arrives in natural-log space.  The Gated DeltaNet step (Yang, Kautz,
 *   Hatamizadeh, "Gated Delta Networks", 2024, written here with S as K x V) is
 *
 *       S <- exp(g_t) * S                       (decay)
 *       S <- S + beta_t * k_t (v_t - S^T k_t)^T (delta-rule erase and write,
 *                                                on the decayed state)
 *       o_t = scale * S^T q_t                   (state after token t)
 *
 *   so that S_t = M_t S_{t-1} + beta_t k_t v_t^T with the decayed erase step
 *   M_t = exp(g_t) (I - beta_t k_t k_t^T).
 *
 *   - In-kernel L2 norm (the page's example passes use_qk_l2norm_in_kernel):
 *     x <- x / sqrt(sum x^2 + 1e-6), applied to q and k before use; the scale
 *     (default K^-1/2) multiplies the normalised q.  The TransformerEngine PR
 *     "[PyTorch] Fused GDN attention" (review, "Smaller items") notes that the
 *     order of scale and normalisation is not documented; normalising first
 *     is the only order in which the scale survives.
 *   - Grouped value heads ("HO = max(H, HV)" in the cudnn-frontend PR's
 *     commit notes): v-head h reads q/k head h / (HV / HK).
 *   - Span summary ("Linear Attention", "Summaries"): the end state from a
 *     given start state, and transition = P^T with P = M_T ... M_1, so that
 *     S_final[j][v] = sum_i S_init[i][v] * transition[i][j] + S_span[j][v].
 *   - An empty sequence (start == end) leaves the state as it was and the
 *     transition equal to the identity.
 *   - Gate and beta transforms (the cudnn-frontend PR's commit notes on
 *     gated_delta_net: use_beta_sigmoid_in_kernel, and safe_gate with a_log /
 *     dt_bias, -exp(a_log) * softplus(g + dt_bias), dt_bias zero when absent):
 *     with beta logits given, beta_t = 1 / (1 + exp(-logit_t)); with a_log
 *     given, the gate is g_t = -exp(a_log[h]) * log(1 + exp(g_t + dt_bias[h]))
 *     in place of the natural-log gate.  Both in double precision.
 *   - Gated Delta Product (the "Linear Attention" page, its description of GDP:
 *     q and g one row per token, k, v and beta n rows per token, update-major;
 *     n = 1 is exactly GDN): per token, the decay exp(g_t) once, then the n
 *     delta-rule updates of that token in order, each on the state the previous
 *     one left, then the output from the state after all of them.  The span
 *     transition is the product of the same steps.
 *   - State series ("Linear Attention" page, "States and checkpoints":
 *     checkpoint_every_n_tokens returns the state series, one entry every n
 *     tokens strictly before each sequence end): entry j of a sequence is the
 *     state after its first j n tokens, for every j n < length; entry 0 is the
 *     initial state.
 *
 * Inputs are taken exactly: bf16 bit patterns are widened to double, fp32
 * values are widened to double.  Every sum is a plain left-to-right loop.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "gdn_oracle.h"

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void load_row(const uint16_t *base, int64_t row, int heads, int head, int dim, double *dst)
{
    const uint16_t *src = base + ((int64_t)row * heads + head) * dim;
    for (int i = 0; i < dim; ++i) dst[i] = bf16_bits_to_double(src[i]);
}

/* x <- x / sqrt(sum x^2 + eps) */
static void l2_normalise(double *x, int dim)
{
    double ss = 0.0;
    for (int i = 0; i < dim; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss + GDN_ORACLE_L2_EPS);
    for (int i = 0; i < dim; ++i) x[i] *= r;
}

/* One (sequence, v-head) unit.  Returns 0 on success, -1 on allocation failure. */
static int run_unit(const gdn_oracle_problem *p, int32_t seq, int32_t head,
                    double *o, double *state_out, double *transition_out, double *checkpoints)
{
    const int K = p->head_dim_k, V = p->head_dim_v;
    const int HK = p->num_qk_heads, HV = p->num_v_heads;
    const int hk = head / (HV / HK);
    const int64_t t0 = p->cu_seqlens[seq], t1 = p->cu_seqlens[seq + 1];
    const int want_transition = transition_out != NULL;

    double *S = (double *)calloc((size_t)K * V, sizeof(double));
    double *P = want_transition ? (double *)calloc((size_t)K * K, sizeof(double)) : NULL;
    double *q = (double *)malloc(sizeof(double) * K);
    double *k = (double *)malloc(sizeof(double) * K);
    double *v = (double *)malloc(sizeof(double) * V);
    double *u = (double *)malloc(sizeof(double) * (V > K ? V : K));
    if (!S || (want_transition && !P) || !q || !k || !v || !u) {
        free(S); free(P); free(q); free(k); free(v); free(u);
        return -1;
    }

    if (p->initial_state) {
        const float *s0 = p->initial_state + ((int64_t)seq * HV + head) * (int64_t)K * V;
        for (int64_t i = 0; i < (int64_t)K * V; ++i) S[i] = (double)s0[i];
    }
    if (want_transition)
        for (int i = 0; i < K; ++i) P[(int64_t)i * K + i] = 1.0;

    const int nh = p->num_householder > 1 ? p->num_householder : 1;
    for (int64_t t = t0; t < t1; ++t) {
        if (checkpoints && (t - t0) % p->checkpoint_every == 0)
            memcpy(checkpoints + ((t - t0) / p->checkpoint_every) * (int64_t)K * V, S,
                   sizeof(double) * (size_t)K * V);
        double gt = (double)p->g[t * HV + head];
        if (p->a_log) {
            const double x = gt + (p->dt_bias ? (double)p->dt_bias[head] : 0.0);
            const double softplus = x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
            gt = -exp((double)p->a_log[head]) * softplus;
        }
        const double a = exp(gt);

        /* decay (state and, for the summary, the span operator) */
        for (int64_t i = 0; i < (int64_t)K * V; ++i) S[i] *= a;
        if (want_transition)
            for (int64_t i = 0; i < (int64_t)K * K; ++i) P[i] *= a;

        for (int r = 0; r < nh; ++r) {
            const int64_t row = t * nh + r;   /* update row of k, v and beta */
            load_row(p->k, row, HK, hk, K, k);
            load_row(p->v, row, HV, head, V, v);
            if (p->l2norm) l2_normalise(k, K);
            const double b = p->beta_logit
                                 ? 1.0 / (1.0 + exp(-bf16_bits_to_double(p->beta_logit[row * HV + head])))
                                 : (double)p->beta[row * HV + head];
            /* u = v - S^T k  (S already decayed) */
            for (int j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i) acc += S[(int64_t)i * V + j] * k[i];
                u[j] = v[j] - acc;
            }
            /* S += beta k u^T */
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j) S[(int64_t)i * V + j] += b * k[i] * u[j];
            if (want_transition) {
                /* P <- (I - beta k k^T) P */
                for (int j = 0; j < K; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < K; ++i) acc += k[i] * P[(int64_t)i * K + j];
                    u[j] = acc;
                }
                for (int i = 0; i < K; ++i)
                    for (int j = 0; j < K; ++j) P[(int64_t)i * K + j] -= b * k[i] * u[j];
            }
        }

        if (o) {
            load_row(p->q, t, HK, hk, K, q);
            if (p->l2norm) l2_normalise(q, K);
            double *orow = o + (t - t0) * V;
            for (int j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i) acc += S[(int64_t)i * V + j] * q[i];
                orow[j] = p->scale * acc;
            }
        }
    }

    if (state_out) memcpy(state_out, S, sizeof(double) * (size_t)K * V);
    if (want_transition)
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j) transition_out[(int64_t)i * K + j] = P[(int64_t)j * K + i];

    free(S); free(P); free(q); free(k); free(v); free(u);
    return 0;
}

int gdn_oracle_run(const gdn_oracle_problem *p, int32_t n_units, const int32_t *unit_seq,
                   const int32_t *unit_head, const int64_t *o_offset, double *o,
                   double *state_out, double *transition_out, int num_threads)
{
    if (!p || n_units < 0 || (n_units > 0 && (!unit_seq || !unit_head))) return -2;
    if (p->num_qk_heads <= 0 || p->num_v_heads <= 0 || p->num_v_heads % p->num_qk_heads) return -2;
    if (p->head_dim_k <= 0 || p->head_dim_v <= 0 || !p->k || !p->v || !p->g || (!p->beta && !p->beta_logit)) return -2;
    if (p->dt_bias && !p->a_log) return -2;
    if (p->checkpoint_every < 0 || (p->checkpoint_every > 0 && (!p->checkpoints || !p->checkpoint_offset)))
        return -2;
    if (o && (!p->q || !o_offset)) return -2;
    for (int32_t u = 0; u < n_units; ++u) {
        if (unit_seq[u] < 0 || unit_seq[u] >= p->num_seqs) return -2;
        if (unit_head[u] < 0 || unit_head[u] >= p->num_v_heads) return -2;
        if (p->cu_seqlens[unit_seq[u] + 1] < p->cu_seqlens[unit_seq[u]]) return -2;
    }
    const int64_t kv = (int64_t)p->head_dim_k * p->head_dim_v;
    const int64_t kk = (int64_t)p->head_dim_k * p->head_dim_k;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : 1) reduction(| : failed)
    for (int32_t u = 0; u < n_units; ++u) {
        double *ou = o ? o + o_offset[u] : NULL;
        double *su = state_out ? state_out + u * kv : NULL;
        double *tu = transition_out ? transition_out + u * kk : NULL;
        double *cu_ = p->checkpoint_every > 0 ? p->checkpoints + p->checkpoint_offset[u] : NULL;
        if (run_unit(p, unit_seq[u], unit_head[u], ou, su, tu, cu_) != 0) failed |= 1;
    }
    return failed ? -1 : 0;
}

/*
 * Backward (the "Linear Attention" page: every variant has a full backward; the gradients
 * of q, k, v, g, beta and the initial state).  Reverse-mode differentiation of the token
 * step above, with S_prev the state before token t, a = exp(g_t) and the normalised rows
 * q^, k^:
 *     S' = a S_prev,   u = v - S'^T k^,   S = S' + beta k^ u^T,   o = scale S^T q^
 * Going back from dS (the gradient of the state after token t, starting at d_final):
 *     dS     += scale q^ do^T          dq^    = scale S do
 *     dbeta   = k^T dS u               du     = beta dS^T k^      dv = du
 *     dk^     = beta dS u - S' du      dS'    = dS - k^ du^T
 *     dg      = a (S_prev . dS')       dS_prev = a dS'
 * and through x^ = x / sqrt(sum x^2 + eps):  dx = r (dx^ - x^ (x^ . dx^)), r = 1 / sqrt(..).
 * The states after every token are kept from a forward pass over the unit.
 */
static int run_unit_bwd(const gdn_oracle_problem *p, int32_t seq, int32_t head, const double *d_o,
                        const double *d_final, double *dq, double *dk, double *dv, double *dg,
                        double *dbeta, double *d_init)
{
    const int K = p->head_dim_k, V = p->head_dim_v;
    const int HK = p->num_qk_heads, HV = p->num_v_heads;
    const int hk = head / (HV / HK);
    const int64_t t0 = p->cu_seqlens[seq], len = p->cu_seqlens[seq + 1] - t0;
    const int64_t KV = (int64_t)K * V;

    double *St = (double *)malloc(sizeof(double) * (size_t)((len + 1) * KV));   /* state after token i - 1 */
    double *qh = (double *)malloc(sizeof(double) * (size_t)(len * K + 1));
    double *kh = (double *)malloc(sizeof(double) * (size_t)(len * K + 1));
    double *rq = (double *)malloc(sizeof(double) * (size_t)(len + 1));
    double *rk = (double *)malloc(sizeof(double) * (size_t)(len + 1));
    double *dS = (double *)calloc((size_t)KV, sizeof(double));
    double *Sp = (double *)malloc(sizeof(double) * (size_t)KV);
    double *vv = (double *)malloc(sizeof(double) * (size_t)V);
    double *u = (double *)malloc(sizeof(double) * (size_t)V);
    double *du = (double *)malloc(sizeof(double) * (size_t)V);
    double *dqh = (double *)malloc(sizeof(double) * (size_t)K);
    double *dkh = (double *)malloc(sizeof(double) * (size_t)K);
    if (!St || !qh || !kh || !rq || !rk || !dS || !Sp || !vv || !u || !du || !dqh || !dkh) {
        free(St); free(qh); free(kh); free(rq); free(rk); free(dS); free(Sp); free(vv); free(u); free(du);
        free(dqh); free(dkh);
        return -1;
    }

    /* forward over the unit, keeping every state */
    if (p->initial_state) {
        const float *s0 = p->initial_state + ((int64_t)seq * HV + head) * KV;
        for (int64_t i = 0; i < KV; ++i) St[i] = (double)s0[i];
    } else {
        memset(St, 0, sizeof(double) * (size_t)KV);
    }
    for (int64_t i = 0; i < len; ++i) {
        const int64_t t = t0 + i;
        double *qi = qh + i * K, *ki = kh + i * K;
        load_row(p->q, t, HK, hk, K, qi);
        load_row(p->k, t, HK, hk, K, ki);
        rq[i] = rk[i] = 1.0;
        if (p->l2norm) {
            double sq = 0.0, sk = 0.0;
            for (int c = 0; c < K; ++c) { sq += qi[c] * qi[c]; sk += ki[c] * ki[c]; }
            rq[i] = 1.0 / sqrt(sq + GDN_ORACLE_L2_EPS);
            rk[i] = 1.0 / sqrt(sk + GDN_ORACLE_L2_EPS);
            for (int c = 0; c < K; ++c) { qi[c] *= rq[i]; ki[c] *= rk[i]; }
        }
        const double a = exp((double)p->g[t * HV + head]), b = (double)p->beta[t * HV + head];
        const double *S0 = St + i * KV;
        double *S1 = St + (i + 1) * KV;
        load_row(p->v, t, HV, head, V, vv);
        for (int64_t e = 0; e < KV; ++e) S1[e] = a * S0[e];
        for (int j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int c = 0; c < K; ++c) acc += S1[(int64_t)c * V + j] * ki[c];
            u[j] = vv[j] - acc;
        }
        for (int c = 0; c < K; ++c)
            for (int j = 0; j < V; ++j) S1[(int64_t)c * V + j] += b * ki[c] * u[j];
    }

    /* backward */
    if (d_final) memcpy(dS, d_final, sizeof(double) * (size_t)KV);
    for (int64_t i = len - 1; i >= 0; --i) {
        const int64_t t = t0 + i;
        const double *qi = qh + i * K, *ki = kh + i * K;
        const double a = exp((double)p->g[t * HV + head]), b = (double)p->beta[t * HV + head];
        const double *S0 = St + i * KV, *S1 = St + (i + 1) * KV;
        /* recompute S' and u */
        load_row(p->v, t, HV, head, V, vv);
        for (int64_t e = 0; e < KV; ++e) Sp[e] = a * S0[e];
        for (int j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int c = 0; c < K; ++c) acc += Sp[(int64_t)c * V + j] * ki[c];
            u[j] = vv[j] - acc;
        }
        /* output */
        const double *doi = d_o ? d_o + i * V : NULL;
        for (int c = 0; c < K; ++c) {
            double acc = 0.0;
            if (doi)
                for (int j = 0; j < V; ++j) acc += S1[(int64_t)c * V + j] * doi[j];
            dqh[c] = p->scale * acc;
        }
        if (doi)
            for (int c = 0; c < K; ++c)
                for (int j = 0; j < V; ++j) dS[(int64_t)c * V + j] += p->scale * qi[c] * doi[j];
        /* delta-rule update */
        double db = 0.0;
        for (int c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int j = 0; j < V; ++j) acc += dS[(int64_t)c * V + j] * u[j];
            db += ki[c] * acc;
            dkh[c] = b * acc;
        }
        for (int j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int c = 0; c < K; ++c) acc += dS[(int64_t)c * V + j] * ki[c];
            du[j] = b * acc;
        }
        for (int c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int j = 0; j < V; ++j) acc += Sp[(int64_t)c * V + j] * du[j];
            dkh[c] -= acc;
        }
        for (int c = 0; c < K; ++c)
            for (int j = 0; j < V; ++j) dS[(int64_t)c * V + j] -= ki[c] * du[j];
        /* decay */
        double da = 0.0;
        for (int64_t e = 0; e < KV; ++e) da += S0[e] * dS[e];
        for (int64_t e = 0; e < KV; ++e) dS[e] *= a;
        /* outputs of this token, through the row norms */
        double pq = 0.0, pk = 0.0;
        for (int c = 0; c < K; ++c) { pq += qi[c] * dqh[c]; pk += ki[c] * dkh[c]; }
        for (int c = 0; c < K; ++c) {
            dq[i * K + c] = p->l2norm ? rq[i] * (dqh[c] - qi[c] * pq) : dqh[c];
            dk[i * K + c] = p->l2norm ? rk[i] * (dkh[c] - ki[c] * pk) : dkh[c];
        }
        for (int j = 0; j < V; ++j) dv[i * V + j] = du[j];
        dg[i] = a * da;
        dbeta[i] = db;
    }
    memcpy(d_init, dS, sizeof(double) * (size_t)KV);

    free(St); free(qh); free(kh); free(rq); free(rk); free(dS); free(Sp); free(vv); free(u); free(du);
    free(dqh); free(dkh);
    return 0;
}

int gdn_oracle_backward(const gdn_oracle_problem *p, int32_t n_units, const int32_t *unit_seq,
                        const int32_t *unit_head, const int64_t *tok_offset, const double *d_o,
                        const double *d_final, double *dq, double *dk, double *dv, double *dg,
                        double *dbeta, double *d_init, int num_threads)
{
    if (!p || n_units < 0 || (n_units > 0 && (!unit_seq || !unit_head || !tok_offset))) return -2;
    if (p->num_qk_heads <= 0 || p->num_v_heads <= 0 || p->num_v_heads % p->num_qk_heads) return -2;
    if (p->head_dim_k <= 0 || p->head_dim_v <= 0 || !p->q || !p->k || !p->v || !p->g || !p->beta) return -2;
    if (p->beta_logit || p->a_log || p->num_householder > 1) return -2;   /* plain inputs only */
    if (!dq || !dk || !dv || !dg || !dbeta || !d_init) return -2;
    for (int32_t u = 0; u < n_units; ++u) {
        if (unit_seq[u] < 0 || unit_seq[u] >= p->num_seqs) return -2;
        if (unit_head[u] < 0 || unit_head[u] >= p->num_v_heads) return -2;
        if (p->cu_seqlens[unit_seq[u] + 1] < p->cu_seqlens[unit_seq[u]]) return -2;
    }
    const int K = p->head_dim_k, V = p->head_dim_v;
    const int64_t KV = (int64_t)K * V;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : 1) reduction(| : failed)
    for (int32_t u = 0; u < n_units; ++u) {
        const int64_t r = tok_offset[u];
        if (run_unit_bwd(p, unit_seq[u], unit_head[u], d_o ? d_o + r * V : NULL, d_final ? d_final + u * KV : NULL,
                         dq + r * K, dk + r * K, dv + r * V, dg + r, dbeta + r, d_init + u * KV) != 0)
            failed |= 1;
    }
    return failed ? -1 : 0;
}
