/*
 * fp64 CPU oracle for the Gated DeltaNet forward, span summary and backward.
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

/*
 * Backward of gdn_oracle_run's forward (the plain inputs: beta, the natural-log gate,
 * n = 1), by reverse-mode differentiation of the token recurrence.  Per unit u, its
 * len tokens at row tok_offset[u] of the packed per-unit arrays:
 *   d_o      : [*, V] upstream gradient of o (row tok_offset[u] + i for token i), or NULL
 *   d_final  : [n_units, K, V] upstream gradient of the final state, or NULL
 *   dq, dk   : [*, K] gradients of the raw q and k rows of this unit's v-head (the
 *              caller sums the v-heads that share a q/k head)
 *   dv       : [*, V];  dg, dbeta : [*]
 *   d_init   : [n_units, K, V] gradient of the initial state
 * Returns 0, -1 on allocation failure, -2 on invalid arguments.
 */
int gdn_oracle_backward(const gdn_oracle_problem *p, int32_t n_units, const int32_t *unit_seq,
                        const int32_t *unit_head, const int64_t *tok_offset, const double *d_o,
                        const double *d_final, double *dq, double *dk, double *dv, double *dg,
                        double *dbeta, double *d_init, int num_threads);

#ifdef __cplusplus
}
#endif

#endif
