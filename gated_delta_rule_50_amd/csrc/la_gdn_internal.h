// Internal interface between the C-ABI layer (la_gdn_api.cpp) and the HIP
// kernels (la_gdn_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_gdn.h"

namespace la {

constexpr int kChunk = 64;            // tokens per chunk; chunks restart at every sequence start
constexpr int kSortMax = 8192;        // sequences the scheduler orders longest-first (more: batch order)
constexpr int kFrag = 64 * 16;        // bytes of one MFMA operand fragment (64 lanes x 16 bytes)
constexpr int kScalars = 256;         // fp32 per (chunk, v-head): d[64], sq[64], U~ scales, gl (one fragment)

// Problem description as the kernels see it (element strides, device pointers).
struct Prob {
    int32_t N;
    int64_t T;
    int32_t HK, HV, K, V;
    float scale;
    int32_t l2norm;
    int32_t max_chunks;               // upper bound on chunks: ceil(T nh / 64) + N
    int32_t intra_grid;               // workgroups of the persistent intra-chunk kernel
    int32_t stream_ops;               // the plain forward's and the summary's intra pass writes the
                                      // inter pass's operands with non-temporal stores (set when
                                      // they outgrow the Infinity Cache)
    const __bf16 *q, *k, *v;
    int64_t qst, qsh, kst, ksh, vst, vsh, ost, osh, gst, bst;
    const float *g, *beta;            // beta: fp32, or null when beta16 is set
    const __bf16 *beta16;             // beta logits in bf16 (beta = sigmoid(logit) in the kernel), or null
    const float *a_log, *dt_bias;     // safe gate g = -exp(a_log[h]) softplus(g + dt_bias[h]), or null
    int32_t nh;                       // Householder updates per token (Gated Delta Product; 1: GDN).
                                      // T and cu_seqlens count tokens; k, v and beta have nh update
                                      // rows per token (update-major), q, g and o one row per token;
                                      // the kernels work in update rows, chunks of 64 updates
    float inv_nh;                     // 1 / nh
    int64_t kstu, vstu, bstu;         // nh > 1: element stride between the update rows of one token;
                                      // kst, vst and bst are then token strides (update-major rows:
                                      // kst = nh kstu; token-major [T, nh, H, D] views: any)
    int32_t ck_every;                 // state series every ck_every tokens (a multiple of 64), 0: none
    int32_t ck_fp32;                  // series rows in fp32 (else bf16)
    int32_t ck_quad;                  // fp32 series in the row-quad layout (the backward's own chunk
                                      // states; the public series is row-major)
    void *ck;                         // [ck_cap, HV, K, V] series, sequences in batch order
    int64_t ck_cap;                   // entries the caller allocated
    const int32_t *cu;
    const float *s0;                  // initial / start state or null
    __bf16 *o;                        // forward output or null (summary)
    float *sT;                        // final / end state or null
    float *trans;                     // transition (summary) or null
};

// Workspace regions (carved by the host from the caller's buffer).  The
// per-chunk operands that the intra-chunk pass hands to the inter-chunk pass
// are stored in the lane order of 32 x 32 x 16 MFMA operands, one 16-byte piece
// per lane, so that every fragment is one coalesced 1 KiB load; reductions over
// state rows or tokens are in accumulator order (rows 16 s + 4 hh + i and
// 16 s + 8 + 4 hh + i of step s in slots i and 4 + i).  Chunk ids index the
// chunk table.
struct Ws {
    int32_t *hdr;      // [0] device status, [1] number of chunks
    int4 *seq_info;    // [N]  (start token, length, first chunk id, unused)
    int4 *chunks;      // [max_chunks]  (sequence, start token, length, chunk index in sequence)
    int32_t *order;    // [N]  sequences, longest first (ties: lower index first)
    uint4 *WF;         // [chunk, HV][key half][token tile][step]  -W, W = T diag(beta 2^gam r_k) K, A fragments
    uint4 *PF;         // [chunk, HV][6]  P^T (masked decayed scaled q k^T), B fragments, forward only
    uint2 *UH;         // [chunk, HV][V/32][token tile][4]  U~ = T diag(beta) V as 32 x 32 accumulator
                       // tiles in fp16, four per lane, each tile scaled by 2^(15 - E) (E: the exponent
                       // with the tile's largest magnitude in [2^(E-1), 2^E))
    float *SC;         // [chunk, HV, kScalars]  per token: d = 2^(gam_n - gam) r_k at 0,
                       // sq = scale r_q 2^gam at 64 (forward); gl = 2^gam_n at 192; the U~ tiles'
                       // E - 15 (int bits) at 128 + 2 (value tile) + token tile
    int32_t *cu32;     // [N + 1]  int32 copy of int64 cu_seqlens (when given as int64)
    // backward only (see workspace_layout's `bwd`):
    uint4 *WTF;        // [chunk, HV][K/32 key tiles][4 token steps]  -W^T A fragments (tokens in
                       // accumulator order)
    uint4 *PTF;        // [chunk, HV][3 causal tiles (s, t) = (0,0), (0,1), (1,1)][2]  P^T A fragments
    uint4 *TB;         // [chunk, HV][64 x 64]  T = (I + A)^-1 in bf16, row-major (full backward)
    float *SB;         // [chunk, HV, kScalars]  gam (log2) at 0, r_k at 64, r_q at 128, beta at 192
    float *CK;         // [chunk, HV, K, V]  fp32 state at each chunk's start, row-quad layout (full backward)
    float *DSN;        // [chunk, HV, K, V]  gradient of each chunk's end state, row-quad layout (full backward)
    __bf16 *DU;        // [chunk, HV, 64, V]  gradient of each chunk's U in bf16, row-major (full backward)
    float *DQH, *DKH;  // [T, HV, K]  per value head: gradients of the scaled, normalised q and k rows
                       // (only with HV > HK: head groups to sum)
};

// Byte layout of the workspace; offsets are 256-byte aligned.
// `bwd`: 0 forward or summary; 1 the span summary's state-gradient mirror (the reverse
// pass's operands only); 2 the full backward (the forward's operands, the reverse pass's,
// and the per-chunk states and gradients the backward's intra pass reads).
struct WsLayout {
    size_t hdr, seq_info, chunks, order, WF, PF, UH, SC, cu32, WTF, PTF, TB, SB, CK, DSN, DU, DQH, DKH, total;
};
WsLayout workspace_layout(int64_t N, int64_t T, int64_t HK, int64_t HV, int64_t K, int64_t V,
                          bool summary, int bwd = 0);
Ws carve_workspace(void *base, const WsLayout &L, bool summary);

// Launch-time timing hook: called before and after each kernel with its id.
struct LaunchHook {
    void (*before)(int kernel_id, hipStream_t s, void *ctx);
    void (*after)(int kernel_id, hipStream_t s, void *ctx);
    void *ctx;
};

// Copies int64 cu_seqlens [n] to int32 on `stream`; an entry outside 0 .. INT32_MAX
// becomes -1, which the scheduler's validation reports as malformed cu_seqlens.
hipError_t convert_cu64(const int64_t *src, int32_t *dst, int n, hipStream_t stream);

// Span summary's state-gradient mirror: dS_start from the span's output gradients and
// dS_end (the intra pass in its reverse-operand mode, then the reverse chunk pass), on the
// workspace carved with bwd = 1.  d_out takes p's o strides.
hipError_t run_summary_bwd(const Prob &p, const Ws &w, const __bf16 *d_out, const float *d_end, float *d_start,
                           hipStream_t stream, const LaunchHook *hook);

// The full backward: gradients of the forward for upstream gradients of o and of the final
// states (the recomputed forward, the reverse chunk pass and the backward's intra pass) on
// the workspace carved with bwd = 2.  d_out takes p's o strides; every output is contiguous
// fp32: dq, dk [T, HK, K], dv [T, HV, V], dg, dbeta [T, HV], d_init [N, HV, K, V].
struct BwdArgs {
    const __bf16 *d_out;
    const float *d_final;             // or null (zeros)
    float *dq, *dk, *dv, *dg, *dbeta, *d_init;
    const float *chunk_states;        // the fp32 state at every chunk start, or null (run the forward again)
};
hipError_t run_backward(const Prob &p, const Ws &w, const BwdArgs &a, hipStream_t stream, const LaunchHook *hook);

// Sets the calling thread's error message (la_last_error_message) and returns st.
la_status fail_message(la_status st, const char *msg);

// Enqueues the whole pipeline (scheduler, intra, inter) on `stream`.
hipError_t run_pipeline(const Prob &p, const Ws &w, bool summary, hipStream_t stream,
                        const LaunchHook *hook);

}  // namespace la
