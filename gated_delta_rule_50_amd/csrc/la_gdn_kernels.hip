// HIP kernels (gfx950) of the chunked Gated DeltaNet forward and span summary.
//
// The method (the cuDNN "Linear Attention" page: a recurrent K x V state per
// (sequence, head), evaluated in chunks; the cudnn-frontend PR "Further reduce
// FROST LA CPU overhead + fully support all L2norm, beta, gate fusion": 64-token
// chunks, a chunk-local cumulative gate in the log2 domain, an intra-chunk
// UT/WY solve and an inter-chunk state pass with a 64-wide value block).
//
// Per (sequence, value head) and per chunk of n <= 64 tokens with start state
// S0 (K x V), with r_k, r_q the inverse L2 norms of the raw bf16 rows k, q and
// gam_t the chunk-local inclusive cumsum of g * log2(e):
//   A[t][s] = beta_t 2^(gam_t - gam_s) r_k,t r_k,s (k_t . k_s)   for s < t, else 0
//   T       = (I + A)^-1                       (unit lower triangular)
//   W       = T diag(beta 2^gam r_k) K          U~ = T diag(beta) V
//   U_new   = U~ - W S0
//   O       = diag(scale r_q 2^gam) Q S0 + P U_new,
//             P[t][s] = scale r_q,t r_k,s 2^(gam_t - gam_s) (q_t . k_s)  for s <= t
//   S_n     = 2^(gam_n) S0 + K^T diag(2^(gam_n - gam) r_k) U_new
// Unrolling the token recurrence over a chunk gives exactly these formulas, so
// the chunked result equals the token-by-token one up to rounding.  Every
// exponent above is <= 0, so no factor can overflow.
//
// Three kernels, all on the caller's stream:
//   k_sched     one workgroup: validates cu_seqlens, builds the chunk table and
//               the longest-first order of sequences
//   k_intra     per (chunk, value head): the prologue (row norms r_q, r_k and
//               the chunk-local gate cumsum), A and P on MFMA, T by forward
//               substitution in LDS, W and U~ on MFMA; writes the operands of the
//               inter-chunk pass in MFMA fragment order
//   k_inter     per (sequence, value head, 32 value columns): the sequential chunk
//               loop; S stays in registers as MFMA accumulator tiles
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Operand layout for one 64-lane wave, with
// q4 = lane / 16 and r16 = lane % 16:
//   A (16 x 32): lane holds row r16, reduction slots 8 q4 .. 8 q4 + 7
//   B (32 x 16): lane holds column r16, reduction slots 8 q4 .. 8 q4 + 7
//   C (16 x 16): lane holds column r16, rows 4 q4 .. 4 q4 + 3
// A reduction over 32 rows that are held as two C tiles (rows 16a..16a+15 and
// 16a+16..16a+31) feeds the B operand straight from the accumulators when the
// reduction index is permuted: slot 8 q4 + j is row 4 q4 + j of the first tile
// for j < 4 and row 4 q4 + j - 4 of the second for j >= 4.  The A operand then
// reads the matching columns, 32a + 4 q4 + {0..3} and 32a + 16 + 4 q4 + {0..3}.
// This keeps S and U_new in registers between the products of the chain.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_gdn_internal.h"
#include "la_gdn.h"

namespace la {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(__bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ __bf16 f2bf(float x) { return static_cast<__bf16>(x); }

// Sum of squares of the 8 bf16 values packed in a 16-byte word.
__device__ __forceinline__ float sumsq8(uint4 u)
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(w[i] << 16);
        const float hi = __uint_as_float(w[i] & 0xffff0000u);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
    }
    return s;
}

// Two 8-byte LDS reads: columns c0 + 4 q4 + {0..3} and c0 + 16 + 4 q4 + {0..3}
// of row `row` (row stride `ld` elements): the permuted A operand.
__device__ __forceinline__ bf16x8 lds_a_perm(const __bf16 *base, int ld, int row, int c0, int q4)
{
    const __bf16 *p = base + row * ld + c0 + 4 * q4;
    const uint2 lo = *reinterpret_cast<const uint2 *>(p);
    const uint2 hi = *reinterpret_cast<const uint2 *>(p + 16);
    uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
    return __builtin_bit_cast(bf16x8, u);
}

// One 16-byte LDS read: columns c0 + 8 q4 .. + 7 of row `row`: the plain operand.
__device__ __forceinline__ bf16x8 lds_op(const __bf16 *base, int ld, int row, int c0, int q4)
{
    return *reinterpret_cast<const bf16x8 *>(base + row * ld + c0 + 8 * q4);
}

// Packs two accumulator tiles (rows 4 q4 + j of each) into a permuted B operand.
__device__ __forceinline__ bf16x8 pack_b(f32x4 a, f32x4 b)
{
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[j] = f2bf(a[j]);
        r[4 + j] = f2bf(b[j]);
    }
    return r;
}

// ---------------------------------------------------------------------------
// k_sched: one workgroup of 1024 threads.

__global__ __launch_bounds__(1024) void k_sched(Prob p, Ws w)
{
    __shared__ int s_bad;
    __shared__ int s_scan[1024];
    __shared__ int s_start[kSortMax + 1];    // cu_seqlens, then first chunk ids (N <= kSortMax)
    __shared__ int s_first[kSortMax];
    __shared__ unsigned long long s_keys[kSortMax];
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int N = p.N;
    const bool small = N <= kSortMax;
    if (tid == 0) s_bad = 0;
    if (tid < 16) w.hdr[kZeroOffset / 4 + tid] = 0;   // the zero block rows past a chunk's end load from
    __syncthreads();

    // cu_seqlens must start at 0, never decrease and end at T.
    for (int i = tid; i <= N; i += nt) {
        const int c = p.cu[i];
        bool bad = c < 0 || (int64_t)c > p.T;
        if (i == 0 && c != 0) bad = true;
        if (i == N && (int64_t)c != p.T) bad = true;
        if (i < N && p.cu[i + 1] < c) bad = true;
        if (bad) atomicOr(&s_bad, 1);
        if (small) s_start[i] = c;
    }
    __syncthreads();
    const int bad = s_bad;
    if (tid == 0) w.hdr[0] = bad ? LA_DEVICE_BAD_CU_SEQLENS : LA_DEVICE_OK;

    // Chunk counts and their exclusive scan.
    int carry = 0;
    for (int base = 0; base < N; base += nt) {
        const int i = base + tid;
        int start = 0, len = 0, nc = 0;
        if (i < N && !bad) {
            start = small ? s_start[i] : p.cu[i];
            len = (small ? s_start[i + 1] : p.cu[i + 1]) - start;
            nc = (len + kChunk - 1) / kChunk;
        }
        s_scan[tid] = nc;
        __syncthreads();
        for (int off = 1; off < nt; off <<= 1) {
            const int add = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += add;
            __syncthreads();
        }
        const int first = carry + s_scan[tid] - nc;
        if (i < N) {
            w.seq_info[i] = make_int4(start, len, first, 0);
            if (small) s_first[i] = first;
        }
        carry += s_scan[nt - 1];
        __syncthreads();
    }
    if (tid == 0) w.hdr[1] = carry;

    // Chunk table: chunk c belongs to the last sequence whose first chunk id is <= c
    // (that sequence is never empty, because an empty one shares its id with the next).
    for (int c = tid; c < carry; c += nt) {
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((small ? s_first[mid] : w.seq_info[mid].z) <= c) lo = mid; else hi = mid - 1;
        }
        const int st0 = small ? s_start[lo] : p.cu[lo];
        const int len = (small ? s_start[lo + 1] : p.cu[lo + 1]) - st0;
        const int j = c - (small ? s_first[lo] : w.seq_info[lo].z);
        const int st = st0 + kChunk * j;
        w.chunks[c] = make_int4(lo, st, min(kChunk, st0 + len - st), j);
    }

    // Longest-first order (ties: lower index first), by a bitonic sort in LDS.
    // The order only decides when a sequence's workgroups start, never what they compute.
    if (N <= kSortMax) {
        int npad = 1;
        while (npad < N) npad <<= 1;
        for (int i = tid; i < npad; i += nt) {
            unsigned long long key = ~0ull;
            if (i < N) {
                const uint32_t len = bad ? 0u : (uint32_t)(s_start[i + 1] - s_start[i]);
                key = ((unsigned long long)(0x7fffffffu - len) << 32) | (uint32_t)i;
            }
            s_keys[i] = key;
        }
        __syncthreads();
        for (int kk = 2; kk <= npad; kk <<= 1) {
            for (int j = kk >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < npad; i += nt) {
                    const int ixj = i ^ j;
                    if (ixj > i) {
                        const unsigned long long a = s_keys[i], b = s_keys[ixj];
                        const bool up = (i & kk) == 0;
                        if ((a > b) == up) {
                            s_keys[i] = b;
                            s_keys[ixj] = a;
                        }
                    }
                }
                __syncthreads();
            }
        }
        for (int i = tid; i < N; i += nt) w.order[i] = (int)(s_keys[i] & 0xffffffffull);
    } else {
        for (int i = tid; i < N; i += nt) w.order[i] = i;
    }
}

// ---------------------------------------------------------------------------
// LDS access helpers.  A "permuted A fragment" of a row-major matrix M holds,
// in lane (q4, r16), M[16 m + r16][32 a + 4 q4 + 0..3] and
// M[16 m + r16][32 a + 16 + 4 q4 + 0..3]; an accumulator fragment holds
// C[16 m + 4 q4 + 0..3][16 n + r16].
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i names an
// 8-byte row R[i][0..3] of bf16; lane 4 a + b of the group receives
// R[a][b], R[a + 4][b], R[a + 8][b], R[a + 12][b].  Choosing the rows lets one
// instruction read four consecutive rows of a column-slice, which is what a
// product that reduces over a row-major tile's rows needs.

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

__device__ __forceinline__ uint2 lds_tr(const void *p)
{
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    return __builtin_bit_cast(uint2, r);
}

// B operand reducing over rows: lane (g, r16) gets M[s0 + 8 g + i][c0 + r16], i = 0..7,
// for a row-major bf16 tile with row stride ld (elements; ld * 2 a multiple of 8).
__device__ __forceinline__ bf16x8 lds_b_tr(const __bf16 *base, int ld, int s0, int c0, int lane)
{
    const int g = lane >> 4, rho = lane & 15;
    const __bf16 *p = base + (s0 + 8 * g + (rho >> 2)) * ld + c0 + 4 * (rho & 3);
    const uint2 lo = lds_tr(p), hi = lds_tr(p + 4 * ld);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ uint4 lds_rowperm(const __bf16 *base, int ld, int row, int c0, int q4)
{
    return __builtin_bit_cast(uint4, lds_a_perm(base, ld, row, c0, q4));
}

// Byte offset of element (row, col) (col a multiple of 4) in a 64 x (8 PPR) bf16
// tile stored as 16-byte pieces with the piece index XOR-swizzled by the row.
template <int PPR>
__device__ __forceinline__ int swz(int row, int col)
{
    return (row * PPR + ((col >> 3) ^ (row % PPR))) * 16 + ((col & 7) >> 2) * 8;
}

__device__ __forceinline__ void lds_wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// k_intra: one workgroup of 4 waves per (chunk, value head).
//
// Phase 1 is the prologue (the fused prologue of the cudnn-frontend PR: q/k L2
// norm and the chunk-local gate cumsum, in log2 units): every value it produces
// is consumed in this workgroup or stored with the operands it scales, so it
// runs here rather than as a separate pass over q and k.  Then A and P (MFMA),
// T = (I + A)^-1 (forward substitution, fp32), W and U~ (MFMA; T diag(beta) is
// split into bf16 high and low parts so that U~ keeps fp32 accuracy), and the
// operands of the inter-chunk pass are written in fragment order.

template <int K, int V, bool FWD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_intra(Prob p, Ws w)
{
    constexpr int KP = K + 8;              // row stride of [token][k] bf16 tiles
    constexpr int VP = V + 8;
    constexpr int XP = KP > VP ? KP : VP;
    constexpr int TP = 64 + 8;             // row stride of [token][token] bf16 tiles
    constexpr int AP = 68;                 // row stride of [token][token] fp32 tiles
    constexpr int KPR = K / 8, VPR = V / 8;  // 16-byte pieces per row
    constexpr int NK = 64 * KPR / 256, NV = 64 * VPR / 256;
    constexpr int NA = K / 32;
    // LDS: sK raw k rows | sX q rows, later v rows | sA A^T (fp32) with the solve's
    // scratch, later Tw, Thi, Tlo (bf16) | sT P (bf16), then T (fp32), then W (bf16)
    constexpr int SA_BYTES = (64 * AP * 4 + 7 * 1024 > 3 * 64 * TP * 2) ? 64 * AP * 4 + 7 * 1024 : 3 * 64 * TP * 2;
    __shared__ __attribute__((aligned(16))) __bf16 sK[64 * KP];
    __shared__ __attribute__((aligned(16))) __bf16 sX[64 * XP];
    __shared__ __attribute__((aligned(16))) float sA[SA_BYTES / 4];
    __shared__ __attribute__((aligned(16))) float sT[64 * AP];
    __shared__ float s_rk[64], s_rq[64], s_gam[64], s_beta[64], s_fw[64];
    __bf16 *const sTw = reinterpret_cast<__bf16 *>(sA);
    __bf16 *const sThi = sTw + 64 * TP;
    __bf16 *const sTlo = sThi + 64 * TP;
    __bf16 *const sP = reinterpret_cast<__bf16 *>(sT);
    __bf16 *const sW = reinterpret_cast<__bf16 *>(sT);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q4 = lane >> 4, r16 = lane & 15;
    const int G = p.HV / p.HK;
    const int items = w.hdr[1] * p.HV;      // (chunk, value head) pairs, chunk-major

    // per-thread staging of the next item's rows (prefetched while the current one computes)
    u32x4 kr[NK], qr[NK], vr[NV];
    float gv = 0.f, bv = 0.f;
    auto load_kq = [&](int it) {
        const int4 ch = w.chunks[it / p.HV];
        const int hk_ = (it % p.HV) / G;
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int e = tid + 256 * j, t = e / KPR, pc = e % KPR;
            const int64_t tg = ch.y + t;
            kr[j] = u32x4{0u, 0u, 0u, 0u};
            qr[j] = u32x4{0u, 0u, 0u, 0u};
            if (t < ch.z) {
                kr[j] = *reinterpret_cast<const u32x4 *>(p.k + tg * p.kst + (int64_t)hk_ * p.ksh + 8 * pc);
                if (FWD) qr[j] = *reinterpret_cast<const u32x4 *>(p.q + tg * p.qst + (int64_t)hk_ * p.qsh + 8 * pc);
            }
        }
    };
    auto load_vgb = [&](int it) {
        const int4 ch = w.chunks[it / p.HV];
        const int h_ = it % p.HV;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = tid + 256 * j, t = e / VPR, pc = e % VPR;
            vr[j] = u32x4{0u, 0u, 0u, 0u};
            if (t < ch.z)
                vr[j] = *reinterpret_cast<const u32x4 *>(p.v + (int64_t)(ch.y + t) * p.vst + (int64_t)h_ * p.vsh + 8 * pc);
        }
        gv = 0.f;
        bv = 0.f;
        if (tid < ch.z) {
            gv = p.g[(int64_t)(ch.y + tid) * p.gst + h_];
            bv = p.beta[(int64_t)(ch.y + tid) * p.bst + h_];
        }
    };

    int it = blockIdx.x;
    if (it < items) {
        load_kq(it);
        load_vgb(it);
    }
    for (; it < items; it += gridDim.x) {
        const int next = it + gridDim.x;
        const int c = it / p.HV, h = it % p.HV;
        const int len = w.chunks[c].z;
        const int64_t ch_h = (int64_t)c * p.HV + h;

        // ---- phase 1 (prologue): row norms, gate cumsum; k and q rows into LDS
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int e = tid + 256 * j, t = e / KPR, pc = e % KPR;
            float sk = sumsq8(__builtin_bit_cast(uint4, kr[j]));
            float sq = FWD ? sumsq8(__builtin_bit_cast(uint4, qr[j])) : 0.f;
#pragma unroll
            for (int off = 1; off < KPR; off <<= 1) {
                sk += __shfl_xor(sk, off, KPR);
                if (FWD) sq += __shfl_xor(sq, off, KPR);
            }
            if (pc == 0) {
                const bool ok = t < len;
                s_rk[t] = ok ? (p.l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f) : 0.f;
                s_rq[t] = (ok && FWD) ? (p.l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f) : 0.f;
            }
            *reinterpret_cast<u32x4 *>(sK + t * KP + 8 * pc) = kr[j];
            if (FWD) *reinterpret_cast<u32x4 *>(sX + t * XP + 8 * pc) = qr[j];
        }
        if (wave == 0) {
            // inclusive scan of g * log2(e) over the chunk (zeros past its end)
            float x = gv * kLog2e;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            s_gam[lane] = x;
            s_beta[lane] = bv;
        }
        if (next < items) load_kq(next);      // k, q registers are free again
        __syncthreads();
        if (tid < 64) s_fw[tid] = s_beta[tid] * exp2f(s_gam[tid]) * s_rk[tid];

        // ---- phase 2: A (strictly lower, stored transposed) and P (lower incl. diagonal).
        // Wave m computes row tile m against column tiles n <= m; all operand fragments
        // are read first.
        {
            const int m = wave;
            bf16x8 fa[NA], fq[NA];
#pragma unroll
            for (int kb = 0; kb < NA; ++kb) {
                fa[kb] = lds_op(sK, KP, 16 * m + r16, 32 * kb, q4);
                if (FWD) fq[kb] = lds_op(sX, XP, 16 * m + r16, 32 * kb, q4);
            }
            const float rq4[4] = {s_rq[16 * m + 4 * q4], s_rq[16 * m + 4 * q4 + 1], s_rq[16 * m + 4 * q4 + 2], s_rq[16 * m + 4 * q4 + 3]};
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                f32x4 av = {0.f, 0.f, 0.f, 0.f};
                if (n <= m) {
                    bf16x8 fb[NA];
#pragma unroll
                    for (int kb = 0; kb < NA; ++kb) fb[kb] = lds_op(sK, KP, 16 * n + r16, 32 * kb, q4);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    f32x4 accq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NA; ++kb) {
                        acc = mfma16(fa[kb], fb[kb], acc);
                        if (FWD) accq = mfma16(fq[kb], fb[kb], accq);
                    }
                    const int s = 16 * n + r16;
                    const float gs = s_gam[s], rks = s_rk[s];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 16 * m + 4 * q4 + j;
                        const float dec = exp2f(fminf(s_gam[t] - gs, 0.f));
                        av[j] = (s < t) ? s_beta[t] * dec * s_rk[t] * rks * acc[j] : 0.f;
                        if (FWD) sP[t * TP + s] = f2bf((s <= t) ? p.scale * rq4[j] * rks * dec * accq[j] : 0.f);
                    }
                } else if (FWD) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sP[(16 * m + 4 * q4 + j) * TP + 16 * n + r16] = f2bf(0.f);
                }
                *reinterpret_cast<f32x4 *>(sA + (16 * n + r16) * AP + 16 * m + 4 * q4) = av;
            }
        }
        __syncthreads();

        // ---- phase 2b: P fragments; v rows into sX (q rows are dead)
        if (FWD) {
#pragma unroll
            for (int f2 = 0; f2 < 2; ++f2) {
                const int f = 2 * wave + f2, m = f >> 1, a = f & 1;
                w.PF[(ch_h * 8 + f) * 64 + lane] = lds_rowperm(sP, TP, 16 * m + r16, 32 * a, q4);
            }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = tid + 256 * j, t = e / VPR, pc = e % VPR;
            *reinterpret_cast<u32x4 *>(sX + t * XP + 8 * pc) = vr[j];
        }
        const float gl = s_gam[len - 1];
        if (next < items) load_vgb(next);     // v, g, beta registers are free again
        __syncthreads();

        // ---- phase 3: T = (I + A)^-1 in 16 x 16 blocks.  T is unit lower triangular
        // with diagonal blocks D_i = (I + A_ii)^-1 and, below them,
        //     T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj          (i > j, T_jj = D_j)
        // (block forward substitution).  Wave b inverts D_b by forward substitution
        // (lane c of the first 16 computes column c); then wave j fills block column
        // j, top to bottom.  All in fp32.
        {
            float *sDT = sA + 64 * AP;            // D_i^T, [4][16][16]
            float *sR = sDT + 4 * 256;            // per-wave 16 x 16 scratch
            const int b = wave;
            {
                // D_b by column-oriented forward substitution: once row j is final, it is
                // subtracted from every later row (A^T row j gives A[i][j] for all i).
                const int cc = lane & 15;
                float acc[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = (i == cc) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float tj = acc[j];
                    const float *arow = sA + (16 * b + j) * AP + 16 * b;   // A^T row j: A[i][j] for all i
#pragma unroll
                    for (int i = j + 1; i < 16; ++i) acc[i] = fmaf(-arow[i], tj, acc[i]);
                }
                if (lane < 16) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        sT[(16 * b + i) * AP + 16 * b + cc] = acc[i];
                        sDT[b * 256 + cc * 16 + i] = acc[i];
                    }
                }
            }
            __syncthreads();
            if (wave < 3) {
                const int j = wave;
                const int r4 = lane >> 4, cc = lane & 15;   // this lane: rows 4 r4 .. 4 r4 + 3, column cc
                float *R = sR + wave * 256;
                for (int i = j + 1; i < 4; ++i) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    for (int k = j; k < i; ++k) {
#pragma unroll
                        for (int x0 = 0; x0 < 16; x0 += 8) {
                            f32x4 a4[8];
                            float tk[8];
#pragma unroll
                            for (int x = 0; x < 8; ++x) {
                                a4[x] = *reinterpret_cast<const f32x4 *>(sA + (16 * k + x0 + x) * AP + 16 * i + 4 * r4);
                                tk[x] = sT[(16 * k + x0 + x) * AP + 16 * j + cc];
                            }
#pragma unroll
                            for (int x = 0; x < 8; ++x)
#pragma unroll
                                for (int e = 0; e < 4; ++e) acc[e] = fmaf(a4[x][e], tk[x], acc[e]);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) R[(4 * r4 + e) * 16 + cc] = acc[e];
                    f32x4 tv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int x0 = 0; x0 < 16; x0 += 8) {
                        f32x4 d4[8];
                        float rx[8];
#pragma unroll
                        for (int x = 0; x < 8; ++x) {
                            d4[x] = *reinterpret_cast<const f32x4 *>(sDT + i * 256 + (x0 + x) * 16 + 4 * r4);
                            rx[x] = R[(x0 + x) * 16 + cc];
                        }
#pragma unroll
                        for (int x = 0; x < 8; ++x)
#pragma unroll
                            for (int e = 0; e < 4; ++e) tv[e] = fmaf(-d4[x][e], rx[x], tv[e]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * r4 + e) * AP + 16 * j + cc] = tv[e];
                }
            } else {
                // zeros above the diagonal blocks
                for (int e = lane; e < 6 * 256; e += 64) {
                    const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
                    const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
                    const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
                    sT[(16 * bi + r) * AP + 16 * bj + cc] = 0.f;
                }
            }
        }
        __syncthreads();

        // ---- phase 3b: Tw = T diag(beta 2^gam r_k), T diag(beta) = Thi + Tlo (bf16)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = tid + 256 * j, i = e >> 6, col = e & 63;
            const float tv = sT[i * AP + col];
            const float tu = tv * s_beta[col];
            const __bf16 hi = f2bf(tu);
            sTw[i * TP + col] = f2bf(tv * s_fw[col]);
            sThi[i * TP + col] = hi;
            sTlo[i * TP + col] = f2bf(tu - bf2f(hi));
        }
        __syncthreads();

        // ---- phase 4: W = Tw K (to LDS, bf16) and U~ = Thi V + Tlo V (fp32 fragments)
        {
            const int m = wave;
            const bf16x8 aw0 = lds_op(sTw, TP, 16 * m + r16, 0, q4), aw1 = lds_op(sTw, TP, 16 * m + r16, 32, q4);
            const bf16x8 ah0 = lds_op(sThi, TP, 16 * m + r16, 0, q4), ah1 = lds_op(sThi, TP, 16 * m + r16, 32, q4);
            const bf16x8 al0 = lds_op(sTlo, TP, 16 * m + r16, 0, q4), al1 = lds_op(sTlo, TP, 16 * m + r16, 32, q4);
#pragma unroll
            for (int n = 0; n < K / 16; ++n) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma16(aw0, lds_b_tr(sK, KP, 0, 16 * n, lane), acc);
                acc = mfma16(aw1, lds_b_tr(sK, KP, 32, 16 * n, lane), acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) sW[(16 * m + 4 * q4 + j) * KP + 16 * n + r16] = f2bf(acc[j]);
            }
#pragma unroll
            for (int n = 0; n < V / 16; ++n) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const bf16x8 b0 = lds_b_tr(sX, XP, 0, 16 * n, lane), b1 = lds_b_tr(sX, XP, 32, 16 * n, lane);
                acc = mfma16(ah0, b0, acc);
                acc = mfma16(al0, b0, acc);
                acc = mfma16(ah1, b1, acc);
                acc = mfma16(al1, b1, acc);
                w.UF[((ch_h * (V / 16) + n) * 4 + m) * 64 + lane] = float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
        // per-token factors of the inter-chunk pass
        {
            float v = 0.f;
            const int t = tid & 63;
            const bool ok = t < len;
            if (tid < 64) v = (ok && FWD) ? p.scale * s_rq[t] * exp2f(s_gam[t]) : 0.f;
            else if (tid < 128) v = ok ? exp2f(gl - s_gam[t]) * s_rk[t] : 0.f;
            else if (tid == 128) v = exp2f(gl);
            w.SC[ch_h * kScalars + tid] = v;
        }
        __syncthreads();

        // ---- phase 5: W fragments
        {
            constexpr int FW = 4 * NA;
#pragma unroll
            for (int f2 = 0; f2 < FW / 4; ++f2) {
                const int f = (FW / 4) * wave + f2, m = f / NA, a = f % NA;
                w.WF[(ch_h * FW + f) * 64 + lane] = lds_rowperm(sW, KP, 16 * m + r16, 32 * a, q4);
            }
        }
        __syncthreads();   // sW, sK and the scalars are rewritten by the next item
    }
}

// ---------------------------------------------------------------------------
// k_inter: one workgroup of 2 waves per (sequence, value head, 32 state
// columns); each wave owns 16 columns and keeps them as 8 accumulator tiles.
// The chunk loop is sequential.  Each chunk's operands (W, P and U~ fragments,
// per-token factors, raw q and k tiles) go straight from memory into one of two
// LDS buffers with direct-to-LDS loads issued a chunk ahead; the raw q/k tiles
// are XOR-swizzled (through the choice of source address) so that the
// fragment reads from them are free of bank conflicts.  Rows past a chunk's
// end load from a zero block.  For the summary the state is widened to [S | P]
// (K x (V + K)): the P columns start at the identity and see U~ = 0, so they
// evolve as the product of the decayed erase steps.

template <int K, int V, bool SUMMARY>
struct InterCfg {
    static constexpr bool FWD = !SUMMARY;
    static constexpr int NW = 2, BV = 16 * NW;
    static constexpr int VA = SUMMARY ? V + K : V;
    static constexpr int NT = VA / BV;
    static constexpr int NA = K / 32;
    static constexpr int PPR = K / 8;             // 16-byte pieces per q/k row
    static constexpr int FW = 4 * NA;             // fragments (1 KiB each) per buffer region
    static constexpr int FP = FWD ? 8 : 0;
    static constexpr int FU = 2 * 4;
    static constexpr int FS = 1;
    static constexpr int FQ = FWD ? 64 * PPR / 64 : 0;
    static constexpr int FK = 64 * PPR / 64;
    static constexpr int oW = 0, oP = oW + FW, oU = oP + FP, oS = oU + FU, oQ = oS + FS, oK = oQ + FQ;
    static constexpr int NF = oK + FK;
};

// Per-lane, chunk-invariant parts of the addresses of the raw q/k tile pieces.
template <int K, int V, bool SUMMARY>
struct InterLane {
    uint32_t offk[InterCfg<K, V, SUMMARY>::FK / 2];   // byte offsets from the chunk's first k row
    uint32_t offq[InterCfg<K, V, SUMMARY>::FK / 2];
    int32_t row[InterCfg<K, V, SUMMARY>::FK / 2];     // tile row each piece belongs to
};

template <int K, int V, bool SUMMARY>
__device__ __forceinline__ void inter_lane_init(const Prob &p, int hk, int wave, int lane,
                                                InterLane<K, V, SUMMARY> &L)
{
    using C = InterCfg<K, V, SUMMARY>;
#pragma unroll
    for (int i = 0; i < C::FK / 2; ++i) {
        const int s = (2 * i + wave) * 64 + lane;
        const int row = s / C::PPR, pc = (s % C::PPR) ^ (row % C::PPR);
        L.row[i] = row;
        L.offk[i] = (uint32_t)(2 * (row * p.kst + hk * p.ksh + 8 * pc));
        L.offq[i] = C::FWD ? (uint32_t)(2 * (row * p.qst + hk * p.qsh + 8 * pc)) : 0u;
    }
}

// Issues the direct-to-LDS loads of one chunk's operands into `buf`.  `wave` is
// wave-uniform (read with readfirstlane) so every LDS destination is a scalar.
template <int K, int V, bool SUMMARY>
__device__ __forceinline__ void inter_issue(const Prob &p, const Ws &w, u32x4 *buf, int cid, int start, int len,
                                            int h, int tile, bool ptile, int wave, int lane,
                                            const InterLane<K, V, SUMMARY> &L)
{
    using C = InterCfg<K, V, SUMMARY>;
    const int64_t chh = (int64_t)cid * p.HV + h;
    auto g2l = [&](const void *src, int f) {
        __builtin_amdgcn_global_load_lds((glb_void *)(src), (lds_void *)(buf + f * 64), 16, 0, 0);
    };
    // fragments written by k_intra, already in lane order
    const uint32_t lo16 = (uint32_t)lane * 16u;
    const char *gW = reinterpret_cast<const char *>(w.WF) + (chh * C::FW + wave) * kFrag;
#pragma unroll
    for (int i = 0; i < C::FW / 2; ++i) g2l(gW + lo16 + i * 2 * kFrag, C::oW + 2 * i + wave);
    if (C::FWD) {
        const char *gP = reinterpret_cast<const char *>(w.PF) + (chh * 8 + wave) * kFrag;
#pragma unroll
        for (int i = 0; i < C::FP / 2; ++i) g2l(gP + lo16 + i * 2 * kFrag, C::oP + 2 * i + wave);
    }
    if (!ptile) {
        const char *gU = reinterpret_cast<const char *>(w.UF) + ((chh * (V / 16) + tile * C::NW) * 4 + wave) * kFrag;
#pragma unroll
        for (int i = 0; i < C::FU / 2; ++i) g2l(gU + lo16 + i * 2 * kFrag, C::oU + 2 * i + wave);
    }
    if (wave == 0) g2l(reinterpret_cast<const char *>(w.SC + chh * kScalars) + lo16, C::oS);
    // raw q and k tiles, pieces XOR-swizzled by row; rows past the end read zeros
    const char *kb = reinterpret_cast<const char *>(p.k + (int64_t)start * p.kst);
    const char *qb = C::FWD ? reinterpret_cast<const char *>(p.q + (int64_t)start * p.qst) : nullptr;
    const void *zero = reinterpret_cast<const char *>(w.hdr) + kZeroOffset;
    if (len == kChunk) {
#pragma unroll
        for (int i = 0; i < C::FK / 2; ++i) {
            g2l(kb + L.offk[i], C::oK + 2 * i + wave);
            if (C::FWD) g2l(qb + L.offq[i], C::oQ + 2 * i + wave);
        }
    } else {
#pragma unroll
        for (int i = 0; i < C::FK / 2; ++i) {
            const bool ok = L.row[i] < len;
            g2l(ok ? (const void *)(kb + L.offk[i]) : zero, C::oK + 2 * i + wave);
            if (C::FWD) g2l(ok ? (const void *)(qb + L.offq[i]) : zero, C::oQ + 2 * i + wave);
        }
    }
}

template <int K, int V, bool SUMMARY>
__device__ __forceinline__ void inter_chunk(const Prob &p, const u32x4 *buf, f32x4 (&S)[K / 16], bool ptile,
                                            int wave, int lane, f32x4 (&O)[4])
{
    using C = InterCfg<K, V, SUMMARY>;
    constexpr int NA = C::NA;
    const int q4 = lane >> 4, r16 = lane & 15;
    const float *sc = reinterpret_cast<const float *>(buf + C::oS * 64);
    const char *tq = reinterpret_cast<const char *>(buf + C::oQ * 64);
    const char *tk = reinterpret_cast<const char *>(buf + C::oK * 64);

    // ---- all LDS reads of the chunk first (independent of S), so their latency
    // overlaps instead of stalling each product
    const int g = q4, rho = r16;
    bf16x8 Wf[4][NA], Qf[4][NA], Kf[K / 16][2], Pf[4][2];
    f32x4 Ut[4], d4[4], sq4[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            Wf[m][a] = __builtin_bit_cast(bf16x8, buf[(C::oW + m * NA + a) * 64 + lane]);
            if (C::FWD) {
                const int row = 16 * m + r16, c0 = 32 * a + 4 * q4;
                const uint2 lo = *reinterpret_cast<const uint2 *>(tq + swz<C::PPR>(row, c0));
                const uint2 hi = *reinterpret_cast<const uint2 *>(tq + swz<C::PPR>(row, c0 + 16));
                Qf[m][a] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        Ut[m] = ptile ? f32x4{0.f, 0.f, 0.f, 0.f}
                      : __builtin_bit_cast(f32x4, buf[(C::oU + wave * 4 + m) * 64 + lane]);
        d4[m] = *reinterpret_cast<const f32x4 *>(sc + 64 + 16 * m + 4 * q4);
        if (C::FWD) sq4[m] = *reinterpret_cast<const f32x4 *>(sc + 16 * m + 4 * q4);
    }
    const float gl = sc[128];
#pragma unroll
    for (int r = 0; r < K / 16; ++r)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            // K^T fragments: transposed reads of the raw k tile
            const int t = 32 * a + 4 * g + (rho >> 2), cc = 16 * r + 4 * (rho & 3);
            const uint2 lo = lds_tr(tk + swz<C::PPR>(t, cc));
            const uint2 hi = lds_tr(tk + swz<C::PPR>(t + 16, cc));
            Kf[r][a] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
    if (C::FWD) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int a = 0; a < 2; ++a) Pf[m][a] = __builtin_bit_cast(bf16x8, buf[(C::oP + 2 * m + a) * 64 + lane]);
    }

    // ---- X = W S and Y = Q S
    bf16x8 Sb[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) Sb[a] = pack_b(S[2 * a], S[2 * a + 1]);
    f32x4 X[4], Y[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        X[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        Y[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            X[m] = mfma16(Wf[m][a], Sb[a], X[m]);
            if (C::FWD) Y[m] = mfma16(Qf[m][a], Sb[a], Y[m]);
        }
    // ---- U_new = U~ - X;  Ud = diag(2^(gam_n - gam) r_k) U_new
    f32x4 Un[4], Ud[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float un = Ut[m][j] - X[m][j];
            Un[m][j] = un;
            Ud[m][j] = d4[m][j] * un;
        }
    const bf16x8 Ud0 = pack_b(Ud[0], Ud[1]), Ud1 = pack_b(Ud[2], Ud[3]);
    // ---- S <- 2^(gam_n) S + K^T Ud
#pragma unroll
    for (int r = 0; r < K / 16; ++r) {
        f32x4 dS = {0.f, 0.f, 0.f, 0.f};
        dS = mfma16(Kf[r][0], Ud0, dS);
        dS = mfma16(Kf[r][1], Ud1, dS);
#pragma unroll
        for (int j = 0; j < 4; ++j) S[r][j] = fmaf(gl, S[r][j], dS[j]);
    }
    // ---- O = diag(scale r_q 2^gam) Q S0 + P U_new
    if (C::FWD) {
        const bf16x8 Ub0 = pack_b(Un[0], Un[1]), Ub1 = pack_b(Un[2], Un[3]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = sq4[m][j] * Y[m][j];
            o = mfma16(Pf[m][0], Ub0, o);
            o = mfma16(Pf[m][1], Ub1, o);
            O[m] = o;
        }
    }
}

template <int K, int V, bool SUMMARY>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_inter(Prob p, Ws w)
{
    using C = InterCfg<K, V, SUMMARY>;
    __shared__ u32x4 buf0[C::NF * 64];
    __shared__ u32x4 buf1[C::NF * 64];

    if (w.hdr[0] != LA_DEVICE_OK) return;
    const int U = p.N * p.HV;
    const int b = blockIdx.x;
    const int grp = b / (8 * C::NT), rem = b % (8 * C::NT);
    const int ug = min(8, U - 8 * grp);
    const int tile = rem / ug;
    const int u = 8 * grp + rem % ug;
    const int n = w.order[u / p.HV];
    const int h = u % p.HV;
    const int hk = h / (p.HV / p.HK);
    const int4 si = w.seq_info[n];
    const int seq_start = si.x, seq_len = si.y, cid0 = si.z;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q4 = lane >> 4, r16 = lane & 15;
    const int tcol0 = tile * C::BV;
    const bool ptile = SUMMARY && tcol0 >= V;
    InterLane<K, V, SUMMARY> L;
    inter_lane_init<K, V, SUMMARY>(p, hk, wave, lane, L);
    const int col = tcol0 + 16 * wave + r16;
    const int64_t unit = (int64_t)n * p.HV + h;

    f32x4 S[K / 16];
    if (!ptile) {
        if (p.s0) {
            const float *s0 = p.s0 + unit * K * V;
#pragma unroll
            for (int r = 0; r < K / 16; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) S[r][j] = s0[(int64_t)(16 * r + 4 * q4 + j) * V + col];
        } else {
#pragma unroll
            for (int r = 0; r < K / 16; ++r) S[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    } else {
        const int pc = col - V;
#pragma unroll
        for (int r = 0; r < K / 16; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[r][j] = (16 * r + 4 * q4 + j == pc) ? 1.f : 0.f;
    }

    const int nch = (seq_len + kChunk - 1) / kChunk;
    f32x4 O[4];
    int o_start = 0, o_len = 0;   // rows of O waiting to be stored (chunk just computed)
    auto store_o = [&]() {
        if (C::FWD && o_len > 0) {
            __bf16 *ob = p.o + (int64_t)o_start * p.ost + (int64_t)h * p.osh + col;
            if (o_len == kChunk) {
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int j = 0; j < 4; ++j) ob[(int64_t)(16 * m + 4 * q4 + j) * p.ost] = f2bf(O[m][j]);
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 16 * m + 4 * q4 + j;
                        if (t < o_len) ob[(int64_t)t * p.ost] = f2bf(O[m][j]);
                    }
            }
        }
        o_len = 0;
    };
    auto chunk_start = [&](int ci) { return seq_start + kChunk * ci; };
    auto chunk_len = [&](int ci) { return min(kChunk, seq_len - kChunk * ci); };

    if (nch > 0)
        inter_issue<K, V, SUMMARY>(p, w, buf0, cid0, chunk_start(0), chunk_len(0), h, tile, ptile, wave, lane, L);
    lds_wait_vm();
    __syncthreads();
    for (int ci = 0; ci < nch; ci += 2) {
        if (ci + 1 < nch)
            inter_issue<K, V, SUMMARY>(p, w, buf1, cid0 + ci + 1, chunk_start(ci + 1), chunk_len(ci + 1), h,
                                       tile, ptile, wave, lane, L);
        store_o();
        inter_chunk<K, V, SUMMARY>(p, buf0, S, ptile, wave, lane, O);
        o_start = chunk_start(ci);
        o_len = chunk_len(ci);
        lds_wait_vm();
        __syncthreads();
        if (ci + 1 >= nch) break;
        if (ci + 2 < nch)
            inter_issue<K, V, SUMMARY>(p, w, buf0, cid0 + ci + 2, chunk_start(ci + 2), chunk_len(ci + 2), h,
                                       tile, ptile, wave, lane, L);
        store_o();
        inter_chunk<K, V, SUMMARY>(p, buf1, S, ptile, wave, lane, O);
        o_start = chunk_start(ci + 1);
        o_len = chunk_len(ci + 1);
        lds_wait_vm();
        __syncthreads();
    }
    store_o();

    if (!ptile) {
        if (p.sT) {
            float *dst = p.sT + unit * K * V;
#pragma unroll
            for (int r = 0; r < K / 16; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[(int64_t)(16 * r + 4 * q4 + j) * V + col] = S[r][j];
        }
    } else {
        // transition[i][j] = P[j][i]: P column pc is transition row pc
        const int pc = col - V;
        float *dst = p.trans + (unit * K + pc) * K;
#pragma unroll
        for (int r = 0; r < K / 16; ++r) *reinterpret_cast<f32x4 *>(dst + 16 * r + 4 * q4) = S[r];
    }
}

// ---------------------------------------------------------------------------
// Host-side launch sequence.

namespace {

template <int K, int V, bool SUMMARY>
hipError_t launch_all(const Prob &p, const Ws &w, hipStream_t s, const LaunchHook *hook)
{
    auto before = [&](int id) { if (hook) hook->before(id, s, hook->ctx); };
    auto after = [&](int id) { if (hook) hook->after(id, s, hook->ctx); };

    before(LA_KERNEL_SCHED);
    hipLaunchKernelGGL(k_sched, dim3(1), dim3(1024), 0, s, p, w);
    after(LA_KERNEL_SCHED);
    if (p.max_chunks > 0) {
        // persistent: at most two resident workgroups per CU, each walking (chunk, head) items
        const int64_t items = (int64_t)p.max_chunks * p.HV;
        const int grid = (int)(items < p.intra_grid ? items : p.intra_grid);
        before(LA_KERNEL_INTRA);
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_intra<K, V, !SUMMARY>), dim3(grid), dim3(256), 0, s, p, w);
        after(LA_KERNEL_INTRA);
    }
    const int64_t blocks = (int64_t)p.N * p.HV * InterCfg<K, V, SUMMARY>::NT;
    if (blocks > 0) {
        before(LA_KERNEL_INTER);
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter<K, V, SUMMARY>), dim3((unsigned)blocks), dim3(128), 0, s, p, w);
        after(LA_KERNEL_INTER);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t run_pipeline(const Prob &p, const Ws &w, bool summary, hipStream_t s, const LaunchHook *hook)
{
    const int K = p.K, V = p.V;
#define LA_DISPATCH(KK, VV)                                                                  \
    if (K == KK && V == VV)                                                                  \
        return summary ? launch_all<KK, VV, true>(p, w, s, hook) : launch_all<KK, VV, false>(p, w, s, hook);
    LA_DISPATCH(64, 64)
    LA_DISPATCH(64, 128)
    LA_DISPATCH(128, 64)
    LA_DISPATCH(128, 128)
#undef LA_DISPATCH
    return hipErrorInvalidValue;
}

}  // namespace la
