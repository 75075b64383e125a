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
// Four kernels, all on the caller's stream:
//   k_sched     one workgroup: validates cu_seqlens, builds the chunk table and
//               the longest-first order of sequences
//   k_prologue  per chunk: r_q, r_k (row norms) and the chunk-local gate cumsum
//   k_intra     per (chunk, value head): A and P on MFMA, T by forward
//               substitution in LDS, W on MFMA, T diag(beta) split into bf16 hi/lo
//   k_inter     per (sequence, value head, value tile): the sequential chunk
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
    __shared__ unsigned long long s_keys[kSortMax];
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int N = p.N;
    if (tid == 0) s_bad = 0;
    __syncthreads();

    // cu_seqlens must start at 0, never decrease and end at T.
    for (int i = tid; i <= N; i += nt) {
        const int c = p.cu[i];
        bool bad = c < 0 || (int64_t)c > p.T;
        if (i == 0 && c != 0) bad = true;
        if (i == N && (int64_t)c != p.T) bad = true;
        if (i < N && p.cu[i + 1] < c) bad = true;
        if (bad) atomicOr(&s_bad, 1);
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
            start = p.cu[i];
            len = p.cu[i + 1] - start;
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
        if (i < N) w.seq_info[i] = make_int4(start, len, carry + s_scan[tid] - nc, 0);
        carry += s_scan[nt - 1];
        __syncthreads();
    }
    if (tid == 0) w.hdr[1] = carry;
    __syncthreads();

    // Chunk table: chunk c belongs to the last sequence whose first chunk id is <= c
    // (that sequence is never empty, because an empty one shares its id with the next).
    for (int c = tid; c < carry; c += nt) {
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (w.seq_info[mid].z <= c) lo = mid; else hi = mid - 1;
        }
        const int4 si = w.seq_info[lo];
        const int j = c - si.z;
        const int st = si.x + kChunk * j;
        w.chunks[c] = make_int4(lo, st, min(kChunk, si.x + si.y - st), j);
    }

    // Longest-first order (ties: lower index first), by a bitonic sort in LDS.
    // The order only decides when a sequence's workgroups start, never what they compute.
    if (N <= kSortMax) {
        int npad = 1;
        while (npad < N) npad <<= 1;
        for (int i = tid; i < npad; i += nt) {
            unsigned long long key = ~0ull;
            if (i < N) {
                const uint32_t len = bad ? 0u : (uint32_t)(p.cu[i + 1] - p.cu[i]);
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
// k_prologue: one workgroup of 256 threads per chunk.

template <int K>
__global__ __launch_bounds__(256) void k_prologue(Prob p, Ws w)
{
    const int c = blockIdx.x;
    if (c >= w.hdr[1]) return;
    const int4 ch = w.chunks[c];
    const int start = ch.y, len = ch.z;
    const int HK = p.HK, HV = p.HV;
    const int rows = len * HK;
    const int nq = p.q ? rows : 0;
    for (int r = threadIdx.x; r < rows + nq; r += blockDim.x) {
        const bool isq = r >= rows;
        const int rr = isq ? r - rows : r;
        const int64_t t = start + rr / HK;
        const int hk = rr % HK;
        const __bf16 *src = isq ? p.q + t * p.qst + hk * p.qsh : p.k + t * p.kst + hk * p.ksh;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < K; i += 8) ss += sumsq8(*reinterpret_cast<const uint4 *>(src + i));
        const float inv = p.l2norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
        (isq ? w.rq : w.rk)[t * HK + hk] = inv;
    }
    for (int h = threadIdx.x; h < HV; h += blockDim.x) {
        float acc = 0.f;
        for (int i = 0; i < len; ++i) {
            const int64_t t = start + i;
            acc = fmaf(p.g[t * p.gst + h], kLog2e, acc);
            w.gam[t * HV + h] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// k_intra: one workgroup of 4 waves per (chunk, value head).

template <int K, bool FWD>
__global__ __launch_bounds__(256) void k_intra(Prob p, Ws w)
{
    constexpr int KP = K + 8;    // row stride (elements) of row-major [token][k] tiles
    constexpr int TP = 64 + 8;   // row stride of [*][token] tiles
    constexpr int AP = 68;       // row stride of the fp32 A^T and T tiles
    __shared__ __attribute__((aligned(16))) __bf16 sK[64 * KP];
    __shared__ __attribute__((aligned(16))) __bf16 sKT[K * TP];
    __shared__ __attribute__((aligned(16))) __bf16 sQ[FWD ? 64 * KP : 8];
    __shared__ __attribute__((aligned(16))) float sAT[64 * AP];
    __shared__ __attribute__((aligned(16))) float sT[64 * AP];
    __shared__ __attribute__((aligned(16))) __bf16 sTw[64 * TP];
    __shared__ float s_rk[64], s_rq[64], s_gam[64], s_beta[64];

    const int c = blockIdx.x, h = blockIdx.y;
    if (c >= w.hdr[1]) return;
    const int4 ch = w.chunks[c];
    const int start = ch.y, len = ch.z;
    const int hk = h / (p.HV / p.HK);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;

    // Stage raw k (row-major and transposed) and q; rows past the chunk are zero.
    for (int e = tid; e < 64 * (K / 8); e += 256) {
        const int t = e / (K / 8), kv = (e % (K / 8)) * 8;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (t < len)
            u = *reinterpret_cast<const uint4 *>(p.k + (int64_t)(start + t) * p.kst + (int64_t)hk * p.ksh + kv);
        *reinterpret_cast<uint4 *>(sK + t * KP + kv) = u;
        const __bf16 *b = reinterpret_cast<const __bf16 *>(&u);
#pragma unroll
        for (int i = 0; i < 8; ++i) sKT[(kv + i) * TP + t] = b[i];
        if (FWD) {
            uint4 uq = make_uint4(0, 0, 0, 0);
            if (t < len)
                uq = *reinterpret_cast<const uint4 *>(p.q + (int64_t)(start + t) * p.qst + (int64_t)hk * p.qsh + kv);
            *reinterpret_cast<uint4 *>(sQ + t * KP + kv) = uq;
        }
    }
    if (tid < 64) {
        const int t = tid;
        const bool ok = t < len;
        const int64_t tg = start + t;
        s_rk[t] = ok ? w.rk[tg * p.HK + hk] : 0.f;
        s_rq[t] = (ok && FWD) ? w.rq[tg * p.HK + hk] : 0.f;
        s_gam[t] = ok ? w.gam[tg * p.HV + h] : 0.f;
        s_beta[t] = ok ? p.beta[tg * p.bst + h] : 0.f;
    }
    __syncthreads();

    // A (strictly lower) and P (lower incl. diagonal): wave m computes row tile m.
    // A is kept transposed in LDS (sAT[s][t] = A[t][s]) so that the solve reads a
    // column of A as contiguous broadcast words.
    {
        const int m = wave;
        for (int n = 0; n < 4; ++n) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            f32x4 accq = {0.f, 0.f, 0.f, 0.f};
            if (n <= m) {
#pragma unroll
                for (int kb = 0; kb < K / 32; ++kb) {
                    const bf16x8 b = lds_op(sK, KP, 16 * n + r16, 32 * kb, q4);
                    acc = mfma16(lds_op(sK, KP, 16 * m + r16, 32 * kb, q4), b, acc);
                    if (FWD) accq = mfma16(lds_op(sQ, KP, 16 * m + r16, 32 * kb, q4), b, accq);
                }
            }
            f32x4 av;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * m + 4 * q4 + j, s = 16 * n + r16;
                const float dec = exp2f(fminf(s_gam[t] - s_gam[s], 0.f));
                av[j] = (s < t) ? s_beta[t] * dec * s_rk[t] * s_rk[s] * acc[j] : 0.f;
                if (FWD && t < len) {
                    const float pv = (s <= t) ? p.scale * s_rq[t] * s_rk[s] * dec * accq[j] : 0.f;
                    w.P[((int64_t)h * p.T + start + t) * 64 + s] = f2bf(pv);
                }
            }
            *reinterpret_cast<f32x4 *>(sAT + (16 * n + r16) * AP + 16 * m + 4 * q4) = av;
        }
    }
    __syncthreads();

    // T = (I + A)^-1 by forward substitution, T[i][c] = [i == c] - sum_{j<i} A[i][j] T[j][c],
    // in 16-row blocks; lane `col` of wave 0 computes column col.  Rows of finished
    // blocks are kept in LDS (sT, fp32).
    if (wave == 0) {
        const int col = lane;
        for (int blk = 0; blk < 4; ++blk) {
            float acc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = (16 * blk + i == col) ? 1.f : 0.f;
            // contributions of the rows of earlier blocks
            for (int j = 0; j < 16 * blk; ++j) {
                const float tj = sT[j * AP + col];
                const f32x4 *arow = reinterpret_cast<const f32x4 *>(sAT + j * AP + 16 * blk);
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 a4 = arow[i4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[4 * i4 + e] = fmaf(-a4[e], tj, acc[4 * i4 + e]);
                }
            }
            // the diagonal block, sequential in its rows
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int j = 16 * blk + jj;
                const float tj = acc[jj];
                sT[j * AP + col] = tj;
                const f32x4 *arow = reinterpret_cast<const f32x4 *>(sAT + j * AP + 16 * blk);
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 a4 = arow[i4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * i4 + e > jj) acc[4 * i4 + e] = fmaf(-a4[e], tj, acc[4 * i4 + e]);
                }
            }
        }
        const float fw = s_beta[col] * exp2f(s_gam[col]) * s_rk[col];
        const float fu = s_beta[col];
        for (int i = 0; i < 64; ++i) {
            const float tv = sT[i * AP + col];
            sTw[i * TP + col] = f2bf(tv * fw);
            if (i < len) {
                const float tu = tv * fu;
                const __bf16 hi = f2bf(tu);
                const __bf16 lo = f2bf(tu - bf2f(hi));
                __bf16 *row = w.TU + ((int64_t)h * p.T + start + i) * 128;
                row[col] = hi;
                row[64 + col] = lo;
            }
        }
    }
    __syncthreads();

    // W = Tw K: wave m computes token rows 16m..16m+15.
    {
        const int m = wave;
        for (int n = 0; n < K / 16; ++n) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                acc = mfma16(lds_op(sTw, TP, 16 * m + r16, 32 * kb, q4),
                             lds_op(sKT, TP, 16 * n + r16, 32 * kb, q4), acc);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * m + 4 * q4 + j;
                if (t < len) w.W[((int64_t)h * p.T + start + t) * K + 16 * n + r16] = f2bf(acc[j]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_inter: one workgroup of NW waves per (sequence, value head, tile of 16 NW
// state columns).  For the summary the state is widened to [S | P] (K x (V + K)):
// the P columns start at the identity and see U~ = 0, so they evolve as the
// product of the decayed erase steps.

template <int K, int V, int NW, bool SUMMARY>
__global__ __launch_bounds__(64 * NW) void k_inter(Prob p, Ws w)
{
    constexpr int BV = 16 * NW;
    constexpr int VA = SUMMARY ? V + K : V;
    constexpr int NT = VA / BV;
    constexpr int KP = K + 8;
    constexpr int TP = 64 + 8;
    constexpr int UP = 128 + 8;
    constexpr bool FWD = !SUMMARY;
    __shared__ __attribute__((aligned(16))) __bf16 sW[64 * KP];
    __shared__ __attribute__((aligned(16))) __bf16 sQ[FWD ? 64 * KP : 8];
    __shared__ __attribute__((aligned(16))) __bf16 sKT[K * TP];
    __shared__ __attribute__((aligned(16))) __bf16 sP[FWD ? 64 * TP : 8];
    __shared__ __attribute__((aligned(16))) __bf16 sTU[64 * UP];
    __shared__ __attribute__((aligned(16))) __bf16 sVT[BV * TP];
    __shared__ float s_sq[64], s_d[64], s_gl;

    if (w.hdr[0] != LA_DEVICE_OK) return;
    const int U = p.N * p.HV;
    const int b = blockIdx.x;
    const int grp = b / (8 * NT), rem = b % (8 * NT);
    const int ug = min(8, U - 8 * grp);
    const int tile = rem / ug;
    const int u = 8 * grp + rem % ug;
    const int n = w.order[u / p.HV];
    const int h = u % p.HV;
    const int hk = h / (p.HV / p.HK);
    const int4 si = w.seq_info[n];
    const int seq_start = si.x, seq_len = si.y;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int tcol0 = tile * BV;                 // first state column of this workgroup
    const bool ptile = SUMMARY && tcol0 >= V;    // the whole tile holds P columns
    const int col = tcol0 + 16 * wave + r16;     // this lane's state column
    const int64_t unit = (int64_t)n * p.HV + h;

    // State tiles: S[r] holds rows 16r + 4q4 + j of column `col`.
    f32x4 S[K / 16];
    if (!ptile) {
        const float *s0 = p.s0 ? p.s0 + unit * K * V : nullptr;
#pragma unroll
        for (int r = 0; r < K / 16; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[r][j] = s0 ? s0[(int64_t)(16 * r + 4 * q4 + j) * V + col] : 0.f;
    } else {
        const int pc = col - V;
#pragma unroll
        for (int r = 0; r < K / 16; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[r][j] = (16 * r + 4 * q4 + j == pc) ? 1.f : 0.f;
    }

    for (int c0 = 0; c0 < seq_len; c0 += kChunk) {
        const int start = seq_start + c0;
        const int len = min(kChunk, seq_len - c0);

        // ---- stage this chunk's operands in LDS (rows past the chunk are zero)
        for (int e = tid; e < 64 * (K / 8); e += 64 * NW) {
            const int t = e / (K / 8), kv = (e % (K / 8)) * 8;
            const bool ok = t < len;
            const int64_t tg = start + t;
            uint4 uw = make_uint4(0, 0, 0, 0), uk = uw, uq = uw;
            if (ok) {
                uw = *reinterpret_cast<const uint4 *>(w.W + ((int64_t)h * p.T + tg) * K + kv);
                uk = *reinterpret_cast<const uint4 *>(p.k + tg * p.kst + (int64_t)hk * p.ksh + kv);
                if (FWD) uq = *reinterpret_cast<const uint4 *>(p.q + tg * p.qst + (int64_t)hk * p.qsh + kv);
            }
            *reinterpret_cast<uint4 *>(sW + t * KP + kv) = uw;
            if (FWD) *reinterpret_cast<uint4 *>(sQ + t * KP + kv) = uq;
            const __bf16 *kb = reinterpret_cast<const __bf16 *>(&uk);
#pragma unroll
            for (int i = 0; i < 8; ++i) sKT[(kv + i) * TP + t] = kb[i];
        }
        for (int e = tid; e < 64 * 16; e += 64 * NW) {
            // TU rows (16 x 16-byte pieces per row) and P rows (8 pieces per row)
            const int t = e / 16, pc = (e % 16) * 8;
            const bool ok = t < len;
            const int64_t tg = start + t;
            uint4 ut = make_uint4(0, 0, 0, 0);
            if (ok) ut = *reinterpret_cast<const uint4 *>(w.TU + ((int64_t)h * p.T + tg) * 128 + pc);
            *reinterpret_cast<uint4 *>(sTU + t * UP + pc) = ut;
            if (FWD && pc < 64) {
                uint4 up = make_uint4(0, 0, 0, 0);
                if (ok) up = *reinterpret_cast<const uint4 *>(w.P + ((int64_t)h * p.T + tg) * 64 + pc);
                *reinterpret_cast<uint4 *>(sP + t * TP + pc) = up;
            }
        }
        if (!ptile) {
            for (int e = tid; e < 64 * (BV / 8); e += 64 * NW) {
                const int t = e / (BV / 8), vv = (e % (BV / 8)) * 8;
                uint4 uv = make_uint4(0, 0, 0, 0);
                if (t < len)
                    uv = *reinterpret_cast<const uint4 *>(p.v + (int64_t)(start + t) * p.vst + (int64_t)h * p.vsh + tcol0 + vv);
                const __bf16 *vb = reinterpret_cast<const __bf16 *>(&uv);
#pragma unroll
                for (int i = 0; i < 8; ++i) sVT[(vv + i) * TP + t] = vb[i];
            }
        }
        if (tid < 64) {
            const int t = tid;
            const float gl = w.gam[(int64_t)(start + len - 1) * p.HV + h];
            float sq = 0.f, d = 0.f;
            if (t < len) {
                const int64_t tg = start + t;
                const float ga = w.gam[tg * p.HV + h];
                d = exp2f(gl - ga) * w.rk[tg * p.HK + hk];
                if (FWD) sq = p.scale * w.rq[tg * p.HK + hk] * exp2f(ga);
            }
            s_sq[t] = sq;
            s_d[t] = d;
            if (t == 0) s_gl = exp2f(gl);
        }
        __syncthreads();

        // ---- per wave: 16 state columns
        // U~ = (T diag(beta))_hi V + (T diag(beta))_lo V   (rows: tokens)
        f32x4 Ut[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) Ut[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!ptile) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 bv = lds_op(sVT, TP, 16 * wave + r16, 32 * kb, q4);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    Ut[m] = mfma16(lds_op(sTU, UP, 16 * m + r16, 32 * kb, q4), bv, Ut[m]);
                    Ut[m] = mfma16(lds_op(sTU, UP, 16 * m + r16, 64 + 32 * kb, q4), bv, Ut[m]);
                }
            }
        }
        // S as bf16 B operands (permuted reduction index)
        bf16x8 Sb[K / 32];
#pragma unroll
        for (int a = 0; a < K / 32; ++a) Sb[a] = pack_b(S[2 * a], S[2 * a + 1]);
        // X = W S and Y = Q S
        f32x4 X[4], Y[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            X[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            Y[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int a = 0; a < K / 32; ++a) {
                X[m] = mfma16(lds_a_perm(sW, KP, 16 * m + r16, 32 * a, q4), Sb[a], X[m]);
                if (FWD) Y[m] = mfma16(lds_a_perm(sQ, KP, 16 * m + r16, 32 * a, q4), Sb[a], Y[m]);
            }
        }
        // U_new = U~ - X; Ud = diag(2^(gam_n - gam) r_k) U_new
        f32x4 Un[4], Ud[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float un = Ut[m][j] - X[m][j];
                Un[m][j] = un;
                Ud[m][j] = s_d[16 * m + 4 * q4 + j] * un;
            }
        const bf16x8 Ud0 = pack_b(Ud[0], Ud[1]), Ud1 = pack_b(Ud[2], Ud[3]);
        // S <- 2^(gam_n) S + K^T Ud
        const float gl = s_gl;
#pragma unroll
        for (int r = 0; r < K / 16; ++r) {
            f32x4 dS = {0.f, 0.f, 0.f, 0.f};
            dS = mfma16(lds_a_perm(sKT, TP, 16 * r + r16, 0, q4), Ud0, dS);
            dS = mfma16(lds_a_perm(sKT, TP, 16 * r + r16, 32, q4), Ud1, dS);
#pragma unroll
            for (int j = 0; j < 4; ++j) S[r][j] = fmaf(gl, S[r][j], dS[j]);
        }
        if (FWD) {
            const bf16x8 Ub0 = pack_b(Un[0], Un[1]), Ub1 = pack_b(Un[2], Un[3]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 O;
#pragma unroll
                for (int j = 0; j < 4; ++j) O[j] = s_sq[16 * m + 4 * q4 + j] * Y[m][j];
                O = mfma16(lds_a_perm(sP, TP, 16 * m + r16, 0, q4), Ub0, O);
                O = mfma16(lds_a_perm(sP, TP, 16 * m + r16, 32, q4), Ub1, O);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * m + 4 * q4 + j;
                    if (t < len) p.o[(int64_t)(start + t) * p.ost + (int64_t)h * p.osh + col] = f2bf(O[j]);
                }
            }
        }
        __syncthreads();
    }

    // ---- write the final (end) state, or the transition for P columns
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
        for (int r = 0; r < K / 16; ++r)
            *reinterpret_cast<f32x4 *>(dst + 16 * r + 4 * q4) = S[r];
    }
}

// ---------------------------------------------------------------------------
// Host-side launch sequence.

namespace {

template <int K, int V, bool SUMMARY>
hipError_t launch_all(const Prob &p, const Ws &w, hipStream_t s, const LaunchHook *hook)
{
    constexpr int NW = 4;
    constexpr int VA = SUMMARY ? V + K : V;
    constexpr int NT = VA / (16 * NW);
    auto before = [&](int id) { if (hook) hook->before(id, s, hook->ctx); };
    auto after = [&](int id) { if (hook) hook->after(id, s, hook->ctx); };

    before(LA_KERNEL_SCHED);
    hipLaunchKernelGGL(k_sched, dim3(1), dim3(1024), 0, s, p, w);
    after(LA_KERNEL_SCHED);
    if (p.max_chunks > 0) {
        before(LA_KERNEL_PROLOGUE);
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_prologue<K>), dim3(p.max_chunks), dim3(256), 0, s, p, w);
        after(LA_KERNEL_PROLOGUE);
        before(LA_KERNEL_INTRA);
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_intra<K, !SUMMARY>), dim3(p.max_chunks, p.HV), dim3(256), 0,
                           s, p, w);
        after(LA_KERNEL_INTRA);
    }
    const int64_t blocks = (int64_t)p.N * p.HV * NT;
    if (blocks > 0) {
        before(LA_KERNEL_INTER);
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter<K, V, NW, SUMMARY>), dim3((unsigned)blocks),
                           dim3(64 * NW), 0, s, p, w);
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
