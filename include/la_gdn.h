/*
 * la_gdn — chunked Gated DeltaNet forward and span summary for AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument named "device" is device memory on the current
 * HIP device; host pointers are named as such.  The caller allocates and frees
 * every buffer, including the workspace, and owns the stream.  The library
 * keeps no pointer after a call returns, allocates no device memory and never
 * synchronises the host with the device (except la_gdn_device_status and
 * la_gdn_profile_read, which exist to do exactly that).  All kernels are
 * enqueued on the caller's stream, so the two compute calls may be captured
 * into a HIP graph.
 *
 * Problem ("Linear Attention" page of the cuDNN docs: opening paragraph,
 * "Layout", "Semantics worth knowing", "Example").  For each sequence n of a
 * packed batch and each value head h the recurrent K x V state S evolves over
 * the sequence's tokens t as
 *       S <- exp(g_t) S;   S <- S + beta_t k_t (v_t - S^T k_t)^T;   o_t = scale S^T q_t
 * (the Gated DeltaNet step), with q and k optionally L2-normalised
 * (x / sqrt(sum x^2 + 1e-6)) before use and scale applied after the norm.
 * Value head h reads q/k head h / (HV / HK).  Tokens are grouped in chunks of
 * 64 that restart at every sequence start, so each sequence's result does not
 * depend on the rest of the batch (the page's "batch_invariant" item), bit
 * for bit.
 *
 * Layouts (the page's "Layout" section: packed THD, strided views with a
 * contiguous innermost axis):
 *   q, k        bf16 [T, HK, K]   strides (q|k)_stride_t, (q|k)_stride_h in elements, innermost 1
 *   v, out      bf16 [T, HV, V]   strides (v|o)_stride_t, (v|o)_stride_h, innermost 1
 *   g, beta     fp32 [T, HV]      stride g_stride_t / beta_stride_t, innermost 1; g is the
 *                                 natural-log gate (decay exp(g) per token)
 *   cu_seqlens  int32 [N + 1]     0 = cu[0] <= cu[1] <= ... <= cu[N] = T
 *   states      fp32 [N, HV, K, V] contiguous
 *   transition  fp32 [N, HV, K, K] contiguous
 * Alignment: q, k, v, out base pointers 16-byte aligned and their outer strides
 * multiples of 8 elements (the library issues 128-bit loads and stores);
 * g, beta, states and transition 4-byte aligned.
 *
 * Errors: host-side checks run before any launch and leave every output
 * untouched; la_last_error_message() names the offending argument.  A
 * malformed cu_seqlens can only be seen on the device: the first kernel
 * detects it, no kernel then writes any output, and la_gdn_device_status()
 * reports LA_DEVICE_BAD_CU_SEQLENS.
 */
#ifndef LA_GDN_H
#define LA_GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad stride or size */
    LA_ERR_UNSUPPORTED = 2,        /* a decline: head dims outside {64, 128}, HV % HK != 0 */
    LA_ERR_WORKSPACE_TOO_SMALL = 3,
    LA_ERR_HIP = 4                 /* a HIP runtime call failed */
} la_status;

/* Device status bits written by the kernels into the workspace. */
#define LA_DEVICE_OK 0
#define LA_DEVICE_BAD_CU_SEQLENS 1

typedef struct {
    int32_t num_seqs;        /* N >= 0; cu_seqlens has N + 1 entries */
    int64_t total_tokens;    /* T >= 0; must equal cu_seqlens[N] (checked on the device) */
    int32_t num_qk_heads;    /* HK >= 1 */
    int32_t num_v_heads;     /* HV >= 1, a multiple of HK; output heads = HV */
    int32_t head_dim_k;      /* K in {64, 128} */
    int32_t head_dim_v;      /* V in {64, 128} */
    float scale;             /* multiplies the (normalised) q; <= 0 means K^-1/2 */
    int64_t q_stride_t, q_stride_h;   /* elements */
    int64_t k_stride_t, k_stride_h;
    int64_t v_stride_t, v_stride_h;
    int64_t o_stride_t, o_stride_h;
    int64_t g_stride_t, beta_stride_t;
} la_gdn_desc;

/*
 * Workspace bytes needed by la_gdn_fwd (is_summary = 0) or la_gdn_summary
 * (is_summary = 1) for this descriptor.  Depends only on N, T, HK, HV, K, V.
 * Returns 0 for an invalid descriptor (see la_last_error_message).
 */
size_t la_gdn_workspace_bytes(const la_gdn_desc *desc, int is_summary);

/*
 * Gated DeltaNet forward ("Linear Attention" page, "Example" and "States and
 * checkpoints": output_final_state, use_qk_l2norm_in_kernel).
 *   q, k, v        device, bf16, layouts above
 *   g, beta        device, fp32 [T, HV]
 *   cu_seqlens     device, int32 [N + 1]
 *   initial_state  device, fp32 [N, HV, K, V], or NULL for zeros
 *   out            device, bf16 [T, HV, V] (written)
 *   final_state    device, fp32 [N, HV, K, V] (written), or NULL to skip
 *   l2norm         nonzero: L2-normalise q and k rows in the kernels
 *   workspace      device, at least la_gdn_workspace_bytes(desc, 0) bytes, 256-byte aligned;
 *                  its contents need no initialisation and are overwritten
 *   stream         HIP stream the kernels are enqueued on
 * An empty sequence (cu[n] == cu[n+1]) gets final = initial (or zeros).
 * N = 0 launches nothing.
 */
la_status la_gdn_fwd(const la_gdn_desc *desc, const void *q, const void *k, const void *v,
                     const float *g, const float *beta, const int32_t *cu_seqlens,
                     const float *initial_state, void *out, float *final_state, int l2norm,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Span summary ("Linear Attention" page, "Summaries"): for every sequence
 * (span) and value head, the end state reached from start_state and the fp32
 * K x K transition, the transpose of the product of the span's decayed erase
 * steps P = M_T ... M_1 with M_t = exp(g_t)(I - beta_t k_t k_t^T), so that
 *     end_state[j][v] = sum_i start_state[i][v] * transition[i][j] + S_span[j][v]
 * where S_span is the end state from a zero start.  q is not used; the q
 * strides of desc are ignored and o strides likewise.
 *   start_state  device, fp32 [N, HV, K, V], or NULL for zeros
 *   end_state    device, fp32 [N, HV, K, V] (written)
 *   transition   device, fp32 [N, HV, K, K] (written)
 * An empty span gets end = start (or zeros) and transition = I.
 */
la_status la_gdn_summary(const la_gdn_desc *desc, const void *k, const void *v, const float *g,
                         const float *beta, const int32_t *cu_seqlens, const float *start_state,
                         float *end_state, float *transition, int l2norm, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * Options of the extended calls.
 *
 * Gate and beta transforms fused into the kernels (the cudnn-frontend pull
 * request "Further reduce FROST LA CPU overhead + fully support all L2norm,
 * beta, gate fusion", commit notes on gated_delta_net: use_beta_sigmoid_in_kernel,
 * and safe_gate with a_log / dt_bias, computing -exp(a_log) * softplus(g + dt_bias)
 * with a zero dt_bias when none is given; beta arrives in the io dtype under the
 * in-kernel sigmoid, else in fp32):
 *   beta_sigmoid  nonzero: `beta` is bf16 [T, HV] logits (stride beta_stride_t,
 *                 2-byte aligned) and the kernels use beta = 1 / (1 + exp(-logit));
 *                 zero: `beta` is fp32 [T, HV] as for la_gdn_fwd
 *   a_log         device, fp32 [HV], or NULL for the plain natural-log gate; when
 *                 given, `g` is the raw gate and the kernels use, per token t and
 *                 value head h, g = -exp(a_log[h]) * log(1 + exp(g_raw[t][h] + dt_bias[h]))
 *   dt_bias       device, fp32 [HV], or NULL for zeros; only with a_log
 * The transforms run in fp32 in the prologue; everything after them is as for
 * la_gdn_fwd / la_gdn_summary.
 *
 * State series (forward only; the "Linear Attention" page, "States and
 * checkpoints": checkpoint_every_n_tokens returns the state series, one entry
 * every n tokens strictly before each sequence end, in the io dtype or, with
 * checkpoint_dtype float32, in fp32):
 *   checkpoint_every_n_tokens  n > 0, a multiple of 64 (the chunk; other values
 *                 are declined with LA_ERR_UNSUPPORTED), or 0 for no series.  Entry
 *                 j of a sequence is the state after its first j n tokens, for
 *                 every j n < length (entry 0 is the initial state); a sequence of
 *                 length L has ceil(L / n) entries, an empty one none
 *   checkpoint_fp32   nonzero: fp32 rows; zero: bf16 rows (round to nearest even)
 *   checkpoints       device, [checkpoint_capacity, HV, K, V] in that dtype, written:
 *                 the entries of sequence 0, then of sequence 1, ...
 *   checkpoint_capacity  entries allocated; entries at or beyond it are not
 *                 written (pass sum over sequences of ceil(L / n))
 *
 * Gated Delta Product (the "Linear Attention" page's description of GDP: q and g
 * one row per token, k, v and beta n rows per token, update-major, and n = 1
 * exactly GDN):
 *   num_householder  n >= 1 (0 means 1).  desc->total_tokens and cu_seqlens count
 *                 tokens; k, v and beta hold n update rows per token, the updates
 *                 of token t being rows t n .. t n + n - 1 (k_stride_t, v_stride_t
 *                 and beta_stride_t step one update row); q, g and out one row per
 *                 token.  Per token the state is decayed once by exp(g_t), then the
 *                 n delta-rule updates run in order, then o_t is read.  The
 *                 workspace is sized by la_gdn_workspace_bytes_ex.  Not combined
 *                 with the state series (LA_ERR_UNSUPPORTED).
 *   householder_token_major  nonzero: k, v and beta come token-major instead
 *                 (the same page: k [T, n, HK, K], v [T, n, HV, V], beta [T, n, HV]
 *                 with the caller's token stride, so that the per-token column slices
 *                 of a joint projection [T, n * H * D], viewed as [T, n, H, D], are read
 *                 in place): update r of token t is at t * k_stride_t +
 *                 r * k_stride_update (likewise v and beta), and k_stride_t, v_stride_t
 *                 and beta_stride_t step one token.  Zero: update-major as above.
 *   k_stride_update, v_stride_update, beta_stride_update  elements between the
 *                 update rows of one token (token-major only).  k and v: multiples
 *                 of 8, covering the heads of a row; the token stride covers all n
 *                 rows; otherwise LA_ERR_INVALID_ARGUMENT.  Token or update strides of
 *                 2^23 elements or more (update-major: the row stride times n) are
 *                 declined with LA_ERR_UNSUPPORTED.
 *
 * Offsets (the "Linear Attention" page lists int32 and int64 cu_seqlens):
 *   cu_seqlens_int64  nonzero: cu_seqlens points at int64 [N + 1] (8-byte aligned,
 *                 else LA_ERR_INVALID_ARGUMENT); a first kernel copies it to int32 in
 *                 the workspace, and an entry outside 0 .. 2^31 - 1 makes the call
 *                 one with malformed cu_seqlens (device status, nothing written).
 *                 Zero: int32 as for la_gdn_fwd.
 */
typedef struct {
    int32_t beta_sigmoid;
    const float *a_log;
    const float *dt_bias;
    int32_t checkpoint_every_n_tokens;
    int32_t checkpoint_fp32;
    void *checkpoints;
    int64_t checkpoint_capacity;
    int32_t num_householder;
    int32_t householder_token_major;
    int64_t k_stride_update;
    int64_t v_stride_update;
    int64_t beta_stride_update;
    int32_t cu_seqlens_int64;
} la_gdn_options;

/* Workspace bytes for la_gdn_fwd_ex / la_gdn_summary_ex with these options (NULL:
   as la_gdn_workspace_bytes); 0 for an invalid descriptor or options. */
size_t la_gdn_workspace_bytes_ex(const la_gdn_desc *desc, int is_summary, const la_gdn_options *options);

/*
 * la_gdn_fwd and la_gdn_summary with the options above (options NULL: the
 * plain calls).  Arguments, errors and outputs are those of the plain calls;
 * `beta` is bf16 or fp32 as options->beta_sigmoid says, and `cu_seqlens` int32 or
 * int64 as options->cu_seqlens_int64 says.  A dt_bias without
 * a_log, a misaligned a_log, dt_bias, beta or checkpoints, or a series without
 * a buffer, is LA_ERR_INVALID_ARGUMENT; a series requested from the summary,
 * or every n that is not a multiple of 64, is LA_ERR_UNSUPPORTED.
 */
la_status la_gdn_fwd_ex(const la_gdn_desc *desc, const void *q, const void *k, const void *v,
                        const float *g, const void *beta, const void *cu_seqlens,
                        const float *initial_state, void *out, float *final_state, int l2norm,
                        const la_gdn_options *options, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);
la_status la_gdn_summary_ex(const la_gdn_desc *desc, const void *k, const void *v, const float *g,
                            const void *beta, const void *cu_seqlens, const float *start_state,
                            float *end_state, float *transition, int l2norm,
                            const la_gdn_options *options, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * The span summary's mirror for the state gradient (the "Linear Attention" page,
 * "Summaries": <op>_summary_bwd, which with the summary implements context
 * parallelism over sequence spans).  For each sequence (span) and value head, with
 * the outputs o_t = scale S_t^T q_t of the forward over the span and
 * L = sum_t <d_out_t, o_t> + <d_end_state, S_end>, returns d_start_state = dL/dS_start:
 * the reverse recurrence D <- d_end_state, then for the span's tokens from last to first
 * D <- exp(g_t) (I - beta_t k_t k_t^T) (D + scale q_t d_out_t^T) (q, k normalised as in
 * the forward).  It does not depend on v or on the start state.
 *   q, k           device, bf16 [T, HK, K] as for la_gdn_fwd
 *   g, beta        device, fp32 [T, HV] (plain natural-log gate, fp32 beta)
 *   cu_seqlens     device, int32 [N + 1]
 *   d_out          device, bf16 [T, HV, V], strides o_stride_t / o_stride_h of desc
 *   d_end_state    device, fp32 [N, HV, K, V], or NULL for zeros
 *   d_start_state  device, fp32 [N, HV, K, V], written
 *   workspace      at least la_gdn_workspace_bytes(desc, 1) bytes, 256-byte aligned
 * Errors as for la_gdn_summary (a malformed cu_seqlens writes nothing and sets the
 * device status).  Evaluated in chunks: the intra pass forms -W^T and P^T per (chunk, head),
 * then the reverse chunk pass of la_gdn_bwd carries the state gradient (one workgroup per
 * (sequence, value head, 32 value columns)).
 */
la_status la_gdn_summary_bwd(const la_gdn_desc *desc, const void *q, const void *k, const float *g,
                             const float *beta, const int32_t *cu_seqlens, const void *d_out,
                             const float *d_end_state, float *d_start_state, int l2norm, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * The full backward of la_gdn_fwd (the "Linear Attention" page: "Every variant has a
 * forward, a full backward"; its "Example" ends in o.sum().backward()).  For upstream
 * gradients d_out of o and d_final_state of the final states, the gradients of
 * L = sum <d_out, o> + sum <d_final_state, final_state> with respect to every input:
 *   q, k, v, g, beta, cu_seqlens, initial_state, l2norm   as for la_gdn_fwd (plain inputs:
 *                  fp32 beta, natural-log gate, int32 cu_seqlens)
 *   d_out          device, bf16 [T, HV, V], strides o_stride_t / o_stride_h of desc
 *   d_final_state  device, fp32 [N, HV, K, V], or NULL for zeros
 *   dq, dk         device, fp32 [T, HK, K] contiguous, 16-byte aligned, written (summed over
 *                  the value heads that share a q/k head, in a fixed order)
 *   dv             device, fp32 [T, HV, V] contiguous, written
 *   dg, dbeta      device, fp32 [T, HV] contiguous, written (dg: gradient of the natural-log gate)
 *   d_initial_state  device, fp32 [N, HV, K, V], written (zero-start inputs still get it)
 *   workspace      at least la_gdn_bwd_workspace_bytes(desc) bytes, 256-byte aligned
 * The forward is run again inside the call (its output is not needed; its state at every
 * chunk start is kept in the workspace), then a reverse pass over the chunks carries the
 * state gradient and a parallel pass forms each chunk's gradients.  Deterministic and batch
 * invariant like the forward.  Errors as for la_gdn_fwd; a malformed cu_seqlens writes
 * nothing and sets the device status.
 */
size_t la_gdn_bwd_workspace_bytes(const la_gdn_desc *desc);
la_status la_gdn_bwd(const la_gdn_desc *desc, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const int32_t *cu_seqlens, const float *initial_state,
                     const void *d_out, const float *d_final_state, float *dq, float *dk, float *dv,
                     float *dg, float *dbeta, float *d_initial_state, int l2norm, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * la_gdn_bwd reusing the forward's states ("Linear Attention" page, "States and
 * checkpoints": the forward can return its state every n tokens for the backward):
 *   chunk_states   device, fp32 [C, HV, K, V], 16-byte aligned, C = sum over sequences of
 *                  ceil(length / 64): the state at the start of every 64-token chunk, in
 *                  sequence order, which la_gdn_fwd_ex writes as its state series with
 *                  checkpoint_every_n_tokens = 64 and fp32 rows from the same inputs and
 *                  initial states; NULL: as la_gdn_bwd (the forward is run again for them)
 * Every other argument as la_gdn_bwd; with the series given, the results are those of
 * la_gdn_bwd bit for bit, and the forward's state pass is not run again.  The series is
 * read, never written, and must not change until the call has run on its stream.
 */
la_status la_gdn_bwd_ex(const la_gdn_desc *desc, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const int32_t *cu_seqlens, const float *initial_state,
                        const float *chunk_states, const void *d_out, const float *d_final_state, float *dq,
                        float *dk, float *dv, float *dg, float *dbeta, float *d_initial_state, int l2norm,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * la_gdn_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Arguments and
 * results are those of la_gdn_fwd (the same checks, kernels and bits) without the
 * workspace: the library's own fixed scratch array serves as it.  That array is 64 MiB
 * per device, held from the first launch on that device until the process ends; a
 * problem whose la_gdn_workspace_bytes(desc, 0) exceeds it is declined with
 * LA_ERR_WORKSPACE_TOO_SMALL before any launch.  The call allocates nothing (no
 * hipMalloc or hipFree, no allocating library routine); its first call on a device
 * looks the array's address up once.  Every call on one GPU shares the array, which
 * keeps the last call's contents (the kernels need nothing in it to start at zero):
 * calls that overlap on one GPU race.  The device status word lives in the array, so
 * la_gdn_device_status cannot read it; a malformed cu_seqlens still writes nothing.
 */
la_status la_gdn_fwd_noalloc(const la_gdn_desc *desc, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const int32_t *cu_seqlens,
                             const float *initial_state, void *out, float *final_state, int l2norm,
                             hipStream_t stream);

/*
 * Reads the status word the last call on this workspace left (LA_DEVICE_*
 * bits).  Synchronises the stream.  Returns -1 if the read itself failed.
 */
int32_t la_gdn_device_status(const void *workspace, hipStream_t stream);

/* Message of the calling thread's last failed call ("" if none). */
const char *la_last_error_message(void);

/*
 * Optional per-kernel timing with HIP events recorded on the caller's stream
 * around each launch.  Off by default; la_gdn_profile_enable(1) turns it on
 * for the calling process and clears the totals.  la_gdn_profile_read waits
 * for the recorded events and returns the summed milliseconds and the launch
 * count of one kernel (ids below).
 */
#define LA_KERNEL_SCHED 0   /* cu_seqlens validation, chunk table, longest-first order (its own
                               kernel only for more than 64 sequences; otherwise k_intra does
                               it and this id counts no launches) */
#define LA_KERNEL_INTRA 1   /* prologue (q/k norms, gate cumsum) + intra-chunk UT/WY */
#define LA_KERNEL_INTER 2   /* sequential inter-chunk state and output pass (any of its variants:
                               forward, summary, with the state series, Gated Delta Product) */
#define LA_KERNEL_BWD_INTRA 3   /* the backward's intra pass and its q/k gradient reduction */
#define LA_KERNEL_COUNT 4
la_status la_gdn_profile_enable(int enable);
la_status la_gdn_profile_read(int32_t kernel_id, double *total_ms, int64_t *launches);
const char *la_gdn_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* LA_GDN_H */
