// Internal interface between the C-ABI layer (la_gdn_api.cpp) and the HIP
// kernels (la_gdn_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kChunk = 64;            // tokens per chunk; chunks restart at every sequence start
constexpr int kSortMax = 8192;        // sequences the scheduler orders longest-first (more: batch order)

// Problem description as the kernels see it (element strides, device pointers).
struct Prob {
    int32_t N;
    int64_t T;
    int32_t HK, HV, K, V;
    float scale;
    int32_t l2norm;
    int32_t max_chunks;               // upper bound on chunks: ceil(T / 64) + N
    const __bf16 *q, *k, *v;
    int64_t qst, qsh, kst, ksh, vst, vsh, ost, osh, gst, bst;
    const float *g, *beta;
    const int32_t *cu;
    const float *s0;                  // initial / start state or null
    __bf16 *o;                        // forward output or null (summary)
    float *sT;                        // final / end state or null
    float *trans;                     // transition (summary) or null
};

// Workspace regions (carved by the host from the caller's buffer).
struct Ws {
    int32_t *hdr;      // [0] device status, [1] number of chunks
    int4 *seq_info;    // [N]  (start token, length, first chunk id, unused)
    int4 *chunks;      // [max_chunks]  (sequence, start token, length, chunk index in sequence)
    int32_t *order;    // [N]  sequences, longest first (ties: lower index first)
    float *rq, *rk;    // [T, HK]  inverse L2 norms of q and k rows (1 when l2norm is off)
    float *gam;        // [T, HV]  chunk-local inclusive cumsum of g * log2(e)
    __bf16 *W;         // [HV, T, K]  W = T diag(beta 2^gam r_k) K per chunk
    __bf16 *TU;        // [HV, T, 128] rows of T diag(beta): bf16 high part | low part
    __bf16 *P;         // [HV, T, 64]  masked, decayed, scaled q k^T per chunk (forward only)
};

// Byte layout of the workspace; offsets are 256-byte aligned.
struct WsLayout {
    size_t hdr, seq_info, chunks, order, rq, rk, gam, W, TU, P, total;
};
WsLayout workspace_layout(int64_t N, int64_t T, int64_t HK, int64_t HV, int64_t K, int64_t V,
                          bool summary);
Ws carve_workspace(void *base, const WsLayout &L, bool summary);

// Launch-time timing hook: called before and after each kernel with its id.
struct LaunchHook {
    void (*before)(int kernel_id, hipStream_t s, void *ctx);
    void (*after)(int kernel_id, hipStream_t s, void *ctx);
    void *ctx;
};

// Enqueues the whole pipeline (scheduler, prologue, intra, inter) on `stream`.
hipError_t run_pipeline(const Prob &p, const Ws &w, bool summary, hipStream_t stream,
                        const LaunchHook *hook);

}  // namespace la
