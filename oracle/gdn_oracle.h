/*
 * fp64 CPU oracle for the Gated DeltaNet forward and span summary.
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU baseline, never by the GPU library.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ORACLE_L2_EPS 1e-6

typedef struct {
    int32_t num_seqs;              /* N */
    int32_t num_qk_heads;          /* HK */
    int32_t num_v_heads;           /* HV, a multiple of HK */
    int32_t head_dim_k;            /* K */
    int32_t head_dim_v;            /* V */
    int32_t l2norm;                /* nonzero: normalise q and k rows */
    double scale;                  /* multiplies the (normalised) q */
    const int32_t *cu_seqlens;     /* [N + 1] */
    const uint16_t *q;             /* bf16 bits, contiguous [T, HK, K]; may be NULL without o */
    const uint16_t *k;             /* bf16 bits, contiguous [T, HK, K] */
    const uint16_t *v;             /* bf16 bits, contiguous [T, HV, V] */
    const float *g;                /* [T, HV], natural-log gate */
    const float *beta;             /* [T, HV] */
    const float *initial_state;    /* [N, HV, K, V] or NULL for zeros */
    /* gate and beta transforms (see gdn_oracle.c); all NULL for the plain inputs */
    const uint16_t *beta_logit;    /* bf16 bits [T, HV]: beta = 1 / (1 + exp(-logit)); replaces beta */
    const float *a_log;            /* [HV]: g = -exp(a_log) * softplus(g + dt_bias) */
    const float *dt_bias;          /* [HV] or NULL for zeros (with a_log only) */
    /* state series: with checkpoint_every = n > 0, unit u writes the state after each
       multiple j n of tokens strictly before its sequence end (j = 0 is the initial state)
       to checkpoints + checkpoint_offset[u] + j K V */
    int32_t checkpoint_every;
    double *checkpoints;
    const int64_t *checkpoint_offset;
    /* Gated Delta Product: n >= 1 Householder updates per token (0 or 1: the plain op).
       k, v and beta (or beta_logit) then have n rows per token, update-major: the updates
       of token t are rows t n .. t n + n - 1; q and g keep one row per token. */
    int32_t num_householder;
} gdn_oracle_problem;

/*
 * Runs the token recurrence for n_units (sequence, v-head) units.
 *   o            : if not NULL, unit u's outputs go to o + o_offset[u] as [len, V]
 *   state_out    : if not NULL, [n_units, K, V] final (end) states
 *   transition_out: if not NULL, [n_units, K, K] transitions (P^T)
 * Units run in parallel on num_threads OpenMP threads.
 * Returns 0, -1 on allocation failure, -2 on invalid arguments.
 */
int gdn_oracle_run(const gdn_oracle_problem *p, int32_t n_units, const int32_t *unit_seq,
                   const int32_t *unit_head, const int64_t *o_offset, double *o,
                   double *state_out, double *transition_out, int num_threads);

#ifdef __cplusplus
}
#endif

#endif
