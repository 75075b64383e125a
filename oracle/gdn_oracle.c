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
