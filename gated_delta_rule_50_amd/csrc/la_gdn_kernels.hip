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
// The kernels, all on the caller's stream:
//   k_cu64      (int64 cu_seqlens only) the int32 copy the other kernels read
//   k_sched     one workgroup, for more than 64 sequences: validates cu_seqlens,
//               builds the chunk table and the longest-first order of sequences
//               (for at most 64, every wave of k_intra maps its own chunks from
//               cu_seqlens and one wave writes the tables)
//   k_intra     per (chunk, value head): the prologue (row norms r_q, r_k, the
//               chunk-local gate cumsum, and optionally the fused beta sigmoid and
//               safe gate), A and P^T on MFMA, T by forward substitution in LDS, W
//               and U~ on MFMA; writes -W, U~ and P^T in MFMA fragment order and the
//               per-token scalars
//   k_inter     per (sequence, value head, 32 value columns): the sequential chunk
//               loop, split over state, output and loader waves; S stays in
//               registers as MFMA accumulator tiles.  Compile-time variants of the
//               same body: k_inter_sum (span summary: no output waves, the state
//               widened by the transition columns), k_inter_ck (with the state
//               series) and k_inter_gdp (Gated Delta Product: q and o rows mapped
//               from update rows to tokens, k rows by token and update) and
//               k_inter_sum_gdp (its summary); k_intra has a Gated Delta Product
//               variant in the same way (k, v and beta rows by token and update).
//               k_inter_wide and k_inter_sum_wide take two 32-column tiles per
//               workgroup, for batches that need more rounds of the CUs
//   backward    k_intra again (both operand sets), k_inter_states (the forward's
//               recurrence again, the fp32 state at every chunk start; two-tile
//               k_inter_states_wide), k_bwd_inter (the reverse chunk pass carrying the
//               state gradient, also the summary's mirror for the state gradient),
//               k_bwd_intra (per (chunk, head) or per (chunk, q/k head group): every
//               gradient of the chunk's algebra) and k_bwd_qk (head-group sums and
//               the row norms' chain rule, where k_bwd_intra does not do them)
//
// MFMA: v_mfma_f32_32x32x16_bf16 for the bf16 products and v_mfma_f32_16x16x4_f32
// for the fp32 block products of the triangular solve (lane layouts with the
// helpers below).  Products that reduce over the rows of an accumulator tile take
// them in accumulator order, so S, U_new and the solve's partial sums feed the
// next product without leaving registers, and the intra-chunk pass writes the
// operands of the inter-chunk pass in that order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_gdn_internal.h"
#include "la_gdn.h"

namespace la {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// 2^x on the hardware exponential (v_exp_f32): one instruction, about 1 ulp; results
// below the normal range flush to zero, and 2^-inf = 0.  The masked entries of the
// decay factors pass -inf, so that masking is a select on the exponent and never a
// branch.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }


__device__ __forceinline__ float bf2f(__bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ __bf16 f2bf(float x) { return static_cast<__bf16>(x); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Sum of squares of the 8 bf16 values packed in a 16-byte word: four two-term bf16 dot
// products (v_dot2c_f32_bf16) accumulated in fp32 (bf16 products are exact in fp32).
__device__ __forceinline__ float sumsq8(uint4 u)
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 x = __builtin_bit_cast(bf16x2, w[i]);
        s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
    }
    return s;
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
// The scheduler for at most 64 sequences, run by every wave of the intra-chunk
// pass instead of a kernel of its own: lane i holds sequence i.  Validates
// cu_seqlens, scans the chunk counts and, in one wave of the grid, writes what
// the inter-chunk pass reads (status, sequence table, longest-first order).

struct SmallMap {
    int start, end, first;   // this lane's sequence: tokens [start, end), first chunk id
    int total;               // chunks of the batch (0 if cu_seqlens is malformed)
};

__device__ __forceinline__ SmallMap small_map(const Prob &p, const Ws &w, bool publish)
{
    const int i = threadIdx.x & 63, N = p.N;
    int start = 0, end = 0;
    bool bad = false;
    if (i < N) {
        // cu_seqlens must start at 0, never decrease and end at T
        start = p.cu[i];
        end = p.cu[i + 1];
        bad = start < 0 || (int64_t)start > p.T || end < start;
        if (i == 0 && start != 0) bad = true;
        if (i == N - 1 && (int64_t)end != p.T) bad = true;
    }
    const bool anybad = __any(bad);
    if (anybad) start = end = 0;
    start *= p.nh;   // update rows from here on (Gated Delta Product: nh per token)
    end *= p.nh;
    const int len = end - start;
    const int nc = (len + kChunk - 1) / kChunk;
    int incl = nc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (i >= off) incl += y;
    }
    SmallMap m;
    m.start = start;
    m.end = end;
    m.first = incl - nc;
    m.total = __shfl(incl, 63, 64);
    if (publish) {
        // longest first, ties by index: the rank of (len, i) in that order
        int rank = 0;
        for (int j = 0; j < N; ++j) {
            const int lj = __shfl(len, j, 64);
            rank += (lj > len || (lj == len && j < i)) ? 1 : 0;
        }
        if (i < N) {
            w.seq_info[i] = make_int4(start, len, m.first, 0);
            w.order[rank] = i;
        }
        if (i == 0) {
            w.hdr[0] = anybad ? LA_DEVICE_BAD_CU_SEQLENS : LA_DEVICE_OK;
            w.hdr[1] = m.total;
        }
    }
    return m;
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
    __syncthreads();

    // cu_seqlens must start at 0, never decrease and end at T.
    for (int i = tid; i <= N; i += nt) {
        const int c = p.cu[i];
        bool bad = c < 0 || (int64_t)c > p.T;
        if (i == 0 && c != 0) bad = true;
        if (i == N && (int64_t)c != p.T) bad = true;
        if (i < N && p.cu[i + 1] < c) bad = true;
        if (bad) atomicOr(&s_bad, 1);
        if (small) s_start[i] = c * p.nh;   // update rows from here on
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
            start = small ? s_start[i] : p.cu[i] * p.nh;
            len = (small ? s_start[i + 1] : p.cu[i + 1] * p.nh) - start;
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
        const int st0 = small ? s_start[lo] : p.cu[lo] * p.nh;
        const int len = (small ? s_start[lo + 1] : p.cu[lo + 1] * p.nh) - st0;
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
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) float lds_float;

__device__ __forceinline__ uint2 lds_tr(const lds_char *p)
{
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ uint2 lds_tr(const void *p)
{
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    return __builtin_bit_cast(uint2, r);
}

// The bf16 operand tiles (64 rows of PPR 16-byte pieces) keep piece j of row r in
// slot j ^ swz_mask(r).  The LDS has 64 banks of 4 bytes, so a 256-byte row (PPR 16)
// covers every bank once and a 128-byte row (PPR 8) half of them.  The mask makes
// both access patterns conflict-free:
//   row reads (one piece of 16 consecutive rows per 16 lanes): the mask is a
//     bijection on those rows (with PPR 8, on the 8 rows of each parity);
//   transposed reads (4 consecutive rows x 4 aligned pieces per 32 lanes): the 4
//     rows' masks differ in the bits above the low two (with PPR 8, the two rows
//     of each parity do), so the 16 (row, piece) pairs land in 16 distinct slots.
// XOR by the row index alone (r % PPR) leaves the transposed reads 4-way conflicted.
template <int PPR>
__device__ __forceinline__ int swz_mask(int row)
{
    if constexpr (PPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else if constexpr (PPR == 8) return (((row >> 1) & 1) << 2) | (((row >> 3) & 1) << 1) | ((row >> 2) & 1);
    else return row % PPR;
}

// Byte offset of element (row, col) (col a multiple of 4) in a 64 x (8 PPR) bf16
// tile stored as 16-byte pieces with the piece index XOR-swizzled by the row.
template <int PPR>
__device__ __forceinline__ int swz(int row, int col)
{
    return (row * PPR + ((col >> 3) ^ swz_mask<PPR>(row))) * 16 + ((col & 7) >> 2) * 8;
}


// ---------------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16, with c = lane % 32 and hh = lane / 32:
//   A (32 x 16): lane holds row c, reduction slots 8 hh .. 8 hh + 7
//   B (16 x 32): lane holds column c, reduction slots 8 hh .. 8 hh + 7
//   C (32 x 32): lane holds column c, rows 8 j + 4 hh + i in register 4 j + i
// A product that reduces over the rows of an accumulator tile takes them in
// register order: step s (s = 0, 1) of a 32-row tile puts rows 16 s + 4 hh + i
// in slots i and rows 16 s + 8 + 4 hh + i in slots 4 + i (i < 4), which are
// registers 8 s .. 8 s + 7 of the lane, so the tile feeds the next product
// without leaving registers ("accumulator order").

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Registers 8 s .. 8 s + 7 of an accumulator tile as a bf16 operand (accumulator order).
__device__ __forceinline__ bf16x8 pack32(const f32x16 &c, int s)
{
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = f2bf(c[8 * s + e]);
    return r;
}

// Sign flip of eight packed bf16 values.
__device__ __forceinline__ uint4 neg_bf16(bf16x8 x)
{
    uint4 u = __builtin_bit_cast(uint4, x);
    u.x ^= 0x80008000u;
    u.y ^= 0x80008000u;
    u.z ^= 0x80008000u;
    u.w ^= 0x80008000u;
    return u;
}

// Workgroup barrier for LDS data exchanged between waves: waits for this wave's
// LDS accesses, then s_barrier (the asm clobbers memory, so no access moves
// across it).  Loads into LDS that are still in flight stay in flight: a
// __syncthreads, or a fence that covers LDS, would wait for them as well.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt, expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

// Buffer resource (four scalar registers) for raw byte-addressed buffer loads.
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
constexpr int kBufferWord3 = 0x00020000;   // raw (unswizzled, unformatted) buffer, CDNA

// Waits until at most N vector memory operations of this wave are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// Buffer loads into LDS and waits shared by both passes.

typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

// A store of one of the inter pass's operands, non-temporal for NT.
template <bool NT, typename T>
__device__ __forceinline__ void st_op(T *dst, T v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, dst);
    else *dst = v;
}

// Lane exchanges within each group of 32 lanes: partner lane c ^ 16 (swizzle, bit mode
// and 0x1f, xor 0x10), c ^ 15 (row mirror), c ^ 7 (half-row mirror), c ^ 2 and c ^ 1 (quad
// permutations).
__device__ __forceinline__ float xch16(float x)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401f));
}
__device__ __forceinline__ float xch15(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, true));
}
__device__ __forceinline__ float xch7(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, true));
}
__device__ __forceinline__ float xch2(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4e, 0xf, 0xf, true));
}
__device__ __forceinline__ float xch1(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xb1, 0xf, 0xf, true));
}

// U~ hand-over in fp16: each 32 x 32 accumulator tile is scaled by 2^(15 - E), E the
// exponent with the tile's largest magnitude in [2^(E-1), 2^E), so that it lands in
// [2^14, 2^15) and every element keeps fp16's 11-bit significand (round to nearest even).
// Returns E - 15, the same in every lane (0 - 15 for an all-zero tile).
__device__ __forceinline__ int f16_tile_shift(const f32x16 &acc)
{
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(acc[e]));
    // the largest over each 32-lane half by lane exchanges (masks 1, 2, 7, 15 and 16 span the
    // half), then over the two halves from lanes 0 and 32
    a = fmaxf(a, xch1(a));
    a = fmaxf(a, xch2(a));
    a = fmaxf(a, xch7(a));
    a = fmaxf(a, xch15(a));
    a = fmaxf(a, xch16(a));
    const float m = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0)),
                          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32)));
    return __builtin_amdgcn_frexp_expf(m) - 15;
}

// Registers 4 j .. 4 j + 3 of a tile, scaled by 2^-sh and rounded to fp16.
__device__ __forceinline__ uint2 f16_pack4(const f32x16 &acc, int j, int sh)
{
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __builtin_amdgcn_ldexpf(acc[4 * j + e], -sh);
    return __builtin_bit_cast(uint2, __builtin_convertvector(x, f16x4));
}

// Row-quad layout of a K x V fp32 state (the backward's chunk-start states and chunk-end
// state gradients): element (row, col) at ((row / 4) V + col) 4 + row % 4, so that rows
// 4 m .. 4 m + 3 of one column, which an accumulator lane holds in four consecutive
// registers, are one 16-byte store, and a 4 x 4 block is four 16-byte loads.
__device__ __forceinline__ int64_t quad_off(int row, int col, int V)
{
    return ((int64_t)(row >> 2) * V + col) * 4 + (row & 3);
}

// Back to fp32 (exact): four fp16 values times 2^sh.
__device__ __forceinline__ f32x4 f16_unpack4(u32x2 h, int sh)
{
    const f32x4 x = __builtin_convertvector(__builtin_bit_cast(f16x4, h), f32x4);
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __builtin_amdgcn_ldexpf(x[e], sh);
    return r;
}
typedef __attribute__((address_space(3))) __bf16 lds_bf16;

__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);   // stride 0: raw byte addressing
    r[2] = (int)bytes;                              // loads at or past this offset read zeros
    r[3] = kBufferWord3;
    return r;
}

// One 16-byte-per-lane buffer load into LDS fragment `f` of `buf` (lane l's 16
// bytes land at fragment byte 16 l).  Written as asm so that the compiler neither
// tracks these loads nor adds waits for them: every wait for them is explicit.
// M0 needs one wait state before the load that uses it.
// The descriptor and the offsets are wave-uniform by contract; they go through readfirstlane
// so that the compiler keeps them in scalar registers, as the instruction needs, also where
// register pressure made it hold them in vector registers.
__device__ __forceinline__ i32x4 uniform_rsrc(i32x4 r)
{
    i32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = __builtin_amdgcn_readfirstlane(r[i]);
    return u;
}

__device__ __forceinline__ void b2l(i32x4 rsrc, lds_u32x4 *buf, int f, uint32_t voff, uint32_t soff)
{
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(buf + f * 64));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(dst), "v"(voff), "s"(uniform_rsrc(rsrc)), "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}

// Waits until at most n (wave-uniform, < 64) vector memory operations of this
// wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait_upto(int n)
{
    if constexpr (N >= 0) {
        if (n == N) vm_wait<N>();
        else vm_wait_upto<N - 1>(n);
    }
}
__device__ __forceinline__ void vm_wait_n(int n)
{
    if (n >= 32) vm_wait_upto<63>(n);
    else if (n >= 16) vm_wait_upto<31>(n);
    else vm_wait_upto<15>(n);
}

// ---------------------------------------------------------------------------
// k_intra: one workgroup of 4 waves per (chunk, value head) item, persistent
// (three workgroups per CU walk the items chunk-major).  Per item:
//   1. k, q, g and beta of the chunk go straight into LDS with buffer loads (rows
//      past the chunk's end are out of the buffer's range and read as zeros; the
//      16-byte pieces of a row are XOR-swizzled by the row, through the choice of
//      source address, so that the operand reads below are free of bank
//      conflicts).  The k rows are issued one item ahead (into sK as soon as the
//      previous item's W products have read it); v lands during 2 and 3.
//   2. the Gram tiles G = K K^T (32 x 32 tiles on or below the diagonal) on bf16
//      MFMA; r_k from the diagonal of G; the chunk-local inclusive gate cumsum gam
//      (log2 units).  Then A = [s < t] beta_t 2^(gam_t - gam_s) r_k,t r_k,s G goes
//      to LDS as A^T, and the per-token scalars of the inter pass (d = 2^(gam_n -
//      gam) r_k, gam, r_k, 2^gam_n) are written out.
//   3. T = (I + A)^-1: the 16 x 16 diagonal blocks D_b by forward substitution
//      (one wave, one lane per column of each block), then block rows 1..3 of
//          T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj
//      on fp32 MFMA (16 x 16 x 4), one block per wave; the sum stays in
//      registers, reduced over in accumulator order by the product with D_i.  T
//      (on and below the diagonal) and A^T (above it) share one fp32 array; the
//      A^T blocks are zeroed once dead, all but block column 3 of rows 0..47.
//   4. -W (from W^T = K^T Tw^T) and U~ = (Thi + Tlo) V on bf16 MFMA, with Tw = T
//      diag(beta 2^gam r_k) and T diag(beta) = Thi + Tlo (bf16) formed in
//      registers; both are written from registers in the inter pass's operand
//      order.

__device__ __forceinline__ void b2l_dword(i32x4 rsrc, lds_float *dst, uint32_t voff)
{
    const uint32_t d = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(dst));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(d), "v"(voff), "s"(uniform_rsrc(rsrc))
                 : "memory", "m0");
}

// Loads a 64-row bf16 tile (rows start at `base`, `rs` bytes apart, `len` of them
// valid) into `dst` as 16-byte pieces swizzled by row; instructions are shared
// round-robin by `nw` waves.
template <int D>
__device__ __forceinline__ void intra_load_tile(lds_u32x4 *dst, const void *base, uint32_t rs, int len, int wave,
                                                int lane, int nw)
{
    constexpr int PPR = D / 8;
    const i32x4 r = make_rsrc(base, (uint32_t)len * rs);
    for (int i = wave; i < PPR; i += nw) {
        const int s = 64 * i + lane, row = s / PPR, pp = s % PPR;
        b2l(r, dst, i, (uint32_t)row * rs + 16u * (uint32_t)(pp ^ swz_mask<PPR>(row)), 0);
    }
}

// Gated Delta Product: the q tile of a chunk of update rows.  Update row start + s
// reads q row (start + s) / nh when it is its token's last update, and zeros
// otherwise (its offset is put past the buffer's range).  `base` points at token
// tb = start / nh, `nrec` bytes of it are in range.
template <int D>
__device__ __forceinline__ void intra_load_qrows(lds_u32x4 *dst, const void *base, uint32_t rs, uint32_t nrec,
                                                 int start, int len, int nh, int tb, int wave, int lane, int nw)
{
    constexpr int PPR = D / 8;
    const i32x4 r = make_rsrc(base, nrec);
    for (int i = wave; i < PPR; i += nw) {
        const int s = 64 * i + lane, row = s / PPR, pp = s % PPR;
        const int u = start + row;
        const bool last = row < len && u % nh == nh - 1;
        b2l(r, dst, i, last ? (uint32_t)(u / nh - tb) * rs + 16u * (uint32_t)(pp ^ swz_mask<PPR>(row)) : nrec, 0);
    }
}

// Gated Delta Product: bytes of q rows in range from token tb on.  A chunk of 64 update
// rows touches at most 64 / nh + 2 tokens, so the range stops at 66 tokens (or the end of
// q): with token strides below 2^24 elements (the host declines larger ones) it fits in
// 32 bits however long the batch is.
__device__ __forceinline__ uint32_t gdp_q_range(const Prob &p, int tb)
{
    const int64_t rows = p.T - tb < 66 ? p.T - tb : 66;
    return (uint32_t)rows * 2u * (uint32_t)p.qst;
}

// Gated Delta Product: element offset of update row tb nh + rel (0 <= rel < 128) from row
// 0 of token tb: rel / nh tokens of stride st and rel % nh updates of stride su (update-major
// rows: st = nh su).  The quotient goes through the reciprocal: (rel + 1/2) / nh lies at
// least 1 / (2 nh) >= 1/128 from an integer, far beyond the float product's rounding.  The
// host keeps 64 st + 64 su below 2^30, so the offset fits in 32 bits.
__device__ __forceinline__ uint32_t upd_off(int rel, int nh, float inv_nh, int st, int su)
{
    const int t = (int)(((float)rel + 0.5f) * inv_nh);
    return (uint32_t)(t * st + (rel - t * nh) * su);
}

// Gated Delta Product: the 64 update rows of a chunk of a bf16 tile (k or v), `len` of them
// valid, from `tok0` = row 0 of the chunk's first token; `phase` = the chunk's first update
// row within that token.  Rows past the end get an offset past the buffer's range and load
// as zeros.  Same LDS layout as intra_load_tile.
template <int D>
__device__ __forceinline__ void intra_load_urows(lds_u32x4 *dst, const __bf16 *tok0, int st, int su, int phase,
                                                 int len, int nh, float inv_nh, int wave, int lane, int nw)
{
    constexpr int PPR = D / 8;
    // (uniform; the float quotient is formed in vector registers)
    const uint32_t nrec = __builtin_amdgcn_readfirstlane(2u * (upd_off(phase + len - 1, nh, inv_nh, st, su) + D));
    const i32x4 r = make_rsrc(tok0, nrec);
    for (int i = wave; i < PPR; i += nw) {
        const int s = 64 * i + lane, row = s / PPR, pp = s % PPR;
        b2l(r, dst, i,
            row < len ? 2u * upd_off(phase + row, nh, inv_nh, st, su) + 16u * (uint32_t)(pp ^ swz_mask<PPR>(row)) : nrec, 0);
    }
}

// 16-byte operand read from a swizzled bf16 tile: row `row`, columns c0 .. c0 + 7 (c0 % 8 == 0).
template <int PPR>
__device__ __forceinline__ bf16x8 lds_row8(const lds_u32x4 *tile, int row, int c0)
{
    return __builtin_bit_cast(bf16x8, tile[row * PPR + ((c0 >> 3) ^ swz_mask<PPR>(row))]);
}

// Transposed reads from a swizzled bf16 tile M (64 rows, PPR pieces per row):
// lane (c, hh) gets M[t0 + 8 hh + e][c0 + c], e = 0..7 (plain order; perm = false)
// or M[t0 + 4 hh + i][c0 + c] in slot i and M[t0 + 8 + 4 hh + i][c0 + c] in slot
// 4 + i (accumulator order; perm = true).
template <int PPR, bool PERM>
__device__ __forceinline__ bf16x8 lds_tr32s(const lds_u32x4 *tile, int t0, int c0, int lane)
{
    const lds_char *b = reinterpret_cast<const lds_char *>(tile);
    const int lam = lane & 15, hh = lane >> 5;
    const int row = t0 + (PERM ? 4 : 8) * hh + (lam >> 2);
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lam & 3);
    const int row2 = row + (PERM ? 8 : 4);
    const uint2 lo = lds_tr(b + swz<PPR>(row, col)), hi = lds_tr(b + swz<PPR>(row2, col));
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// lds_tr32s<PPR, true> with the lane's part of the two addresses precomputed: for t0 a
// multiple of 16 and c0 a multiple of 32, the swizzle mask depends on the lane's row within
// 16 only, and the piece index (c0 / 8 + x) ^ mask splits into a part of c0 and one of the
// lane, so the byte offset is tr_lane_off(...) + 16 PPR t0.  Returns the two offsets.
template <int PPR>
__device__ __forceinline__ uint2 tr_lane_off(int c0, int lane)
{
    const int lam = lane & 15, hh = lane >> 5;
    const int x = 2 * ((lane >> 4) & 1) + ((lam & 3) >> 1), h8 = 8 * (lam & 1);
    uint32_t off[2];
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        const int rr = 4 * hh + (lam >> 2) + 8 * part;      // the row within 16 (accumulator order)
        const int piece = ((c0 >> 3) | x) ^ swz_mask<PPR>(rr);
        off[part] = (uint32_t)((rr * PPR + piece) * 16 + h8);
    }
    return make_uint2(off[0], off[1]);
}

__device__ __forceinline__ bf16x8 lds_tr32s_at(const lds_char *b, uint2 off)
{
    const uint2 lo = lds_tr(b + off.x), hi = lds_tr(b + off.y);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// BW selects what the pass writes for a backward: 0 the forward's operands (plain forward
// and summary); 1 the reverse pass's operands only (-W^T and P^T fragments and the
// scalars, no v: the span summary's state-gradient mirror); 2 both sets, plus T in bf16 and
// the per-token factors (gam, r_k, r_q, beta) for the backward's intra pass.  NT: the
// forward's operands (-W, U~, P^T) are written with non-temporal stores.
template <int K, int V, bool FWD, bool GDP, int BW = 0, bool NT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_intra(Prob p, Ws w)
{
    static_assert(BW == 0 || (FWD && !GDP), "the backward's operands come from the plain forward's pass");
    static_assert(!NT || (BW == 0 && !GDP), "non-temporal operand stores: plain forward and summary");
    constexpr bool WANT_V = BW != 1;                // v, U~ and the forward's -W and P^T
    constexpr int PK = K / 8, PV = V / 8;           // 16-byte pieces per k / v row
    constexpr int DX = K > V ? K : V;
    constexpr int PX = DX / 8;
    constexpr int TS = 68;                          // row stride of the fp32 A^T / T array
    constexpr int NKS = K / 32;                     // reduction steps over a key half (inter pass)
    __shared__ u32x4 sK_[64 * PK];                  // raw k rows, swizzled
    __shared__ u32x4 sX_[64 * PX];                  // raw q rows (forward), then raw v rows, swizzled
    __shared__ float sAT_[64 * TS];                 // A^T above the diagonal, T on and below it
    __shared__ __attribute__((aligned(16))) float sc_[6 * 64];          // per-token scalars
    lds_u32x4 *const sK = (lds_u32x4 *)sK_;
    lds_u32x4 *const sX = (lds_u32x4 *)sX_;
    lds_float *const sAT = (lds_float *)sAT_;
    lds_float *const s_g = (lds_float *)sc_;        // loaded g (0 past the end)
    lds_float *const s_b = s_g + 64;                // loaded beta (0 past the end)
    lds_float *const s_rk = s_g + 128;
    lds_float *const s_rq = s_g + 192;
    lds_float *const s_gam = s_g + 256;
    lds_float *const s_fw = s_g + 320;              // beta 2^gam r_k

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, hh = lane >> 5;
    const int G = p.HV / p.HK;
    // chunk table: from cu_seqlens in registers for at most 64 sequences, else the scheduler's
    const bool small = p.N <= 64;
    SmallMap sm{};
    if (small) sm = small_map(p, w, blockIdx.x == 0 && wave == 0);
    const int items = (small ? sm.total : w.hdr[1]) * p.HV;   // (chunk, value head) pairs, chunk-major

    // Item order: the G value heads that share a q/k head (consecutive items) go to
    // workgroups 8 apart, which the dispatcher places on one XCD, so that their k and q
    // loads share that XCD's L2.  A bijection on the first 8 G floor(groups / 8) items
    // (the rest keep their index); with G = 1 it is the identity.
    const int groups = items / G, full = (groups & ~7) * G;
    struct Item { int ci, h, hk, start, len; };
    auto item_info = [&](int it) {
        int r = it;
        if (G > 1 && it < full) {
            const int u = it >> 3;
            r = __builtin_amdgcn_readfirstlane((8 * (u / G) + (it & 7)) * G + u % G);
        }
        Item x;
        x.ci = __builtin_amdgcn_readfirstlane(r / p.HV);
        x.h = __builtin_amdgcn_readfirstlane(r % p.HV);
        x.hk = __builtin_amdgcn_readfirstlane(x.h / G);
        if (small) {
            // chunk ci belongs to the last sequence whose first chunk id is <= ci (never an
            // empty one: an empty sequence shares its first id with the next)
            const uint64_t owns = __ballot(lane < p.N && sm.first <= x.ci);
            const int n = 63 - __builtin_clzll(owns);
            x.start = __builtin_amdgcn_readfirstlane(__shfl(sm.start, n, 64) + kChunk * (x.ci - __shfl(sm.first, n, 64)));
            x.len = __builtin_amdgcn_readfirstlane(min(kChunk, __shfl(sm.end, n, 64) - x.start));
        } else {
            const int4 ch = w.chunks[x.ci];
            x.start = __builtin_amdgcn_readfirstlane(ch.y);
            x.len = __builtin_amdgcn_readfirstlane(ch.z);
        }
        return x;
    };
    // The k rows of an item into sK.  They are issued one item ahead: for the first item
    // here, for the next one as soon as the W products have read sK, so that their latency
    // overlaps the U~ products and the stores.
    auto issue_k = [&](const Item &x) {
        if (!GDP) {
            intra_load_tile<K>(sK, p.k + (int64_t)x.start * p.kst + (int64_t)x.hk * p.ksh, 2u * (uint32_t)p.kst, x.len,
                               wave, lane, 4);
        } else {
            const int tb = __builtin_amdgcn_readfirstlane(x.start / p.nh);
            intra_load_urows<K>(sK, p.k + (int64_t)tb * p.kst + (int64_t)x.hk * p.ksh, (int)p.kst, (int)p.kstu,
                                x.start - tb * p.nh, x.len, p.nh, p.inv_nh, wave, lane, 4);
        }
    };
    // q (forward), g and beta of an item into LDS, issued one item ahead like k (once the
    // previous item's last reads of sX and the scalars are done); wave 3 also takes the
    // per-lane values that do not go through LDS.
    struct Pre {
        float blogit;   // beta logit of update row `lane` (beta16 only)
        float graw;     // Gated Delta Product: the gate of update row `lane`'s token at its first update
        bool gfirst;    // update row `lane` is its token's first update (always, for GDN)
    };
    Pre pre{0.f, 0.f, true};
    auto issue_qgb = [&](const Item &x) {
        const int start = __builtin_amdgcn_readfirstlane(x.start), len = __builtin_amdgcn_readfirstlane(x.len);
        const int h = __builtin_amdgcn_readfirstlane(x.h), hk = __builtin_amdgcn_readfirstlane(x.hk);
        // Gated Delta Product: the chunk's first token and its first update row within it
        const int tb = GDP ? __builtin_amdgcn_readfirstlane(start / p.nh) : start;
        const int phase = start - tb * p.nh;
        if (FWD) {
            if (!GDP) {
                intra_load_tile<K>(sX, p.q + (int64_t)start * p.qst + (int64_t)hk * p.qsh, 2u * (uint32_t)p.qst,
                                   len, wave, lane, 4);
            } else {
                intra_load_qrows<K>(sX, p.q + (int64_t)tb * p.qst + (int64_t)hk * p.qsh, 2u * (uint32_t)p.qst,
                                    gdp_q_range(p, tb), start, len, p.nh, tb, wave, lane, 4);
            }
        }
        pre.blogit = 0.f;
        pre.graw = 0.f;
        pre.gfirst = true;
        if (wave == 3) {
            if (!GDP) {
                const i32x4 rg = make_rsrc(p.g + (int64_t)start * p.gst + h, (uint32_t)len * 4u * (uint32_t)p.gst);
                b2l_dword(rg, s_g, (uint32_t)lane * 4u * (uint32_t)p.gst);
            } else {
                const int u = start + lane;
                pre.gfirst = u % p.nh == 0;
                if (lane < len && pre.gfirst) pre.graw = p.g[(int64_t)(u / p.nh) * p.gst + h];
            }
            if (!GDP) {
                if (p.beta16) {
                    if (lane < len) pre.blogit = bf2f(p.beta16[(int64_t)(start + lane) * p.bst + h]);
                } else {
                    const i32x4 rb = make_rsrc(p.beta + (int64_t)start * p.bst + h, (uint32_t)len * 4u * (uint32_t)p.bst);
                    b2l_dword(rb, s_b, (uint32_t)lane * 4u * (uint32_t)p.bst);
                }
            } else {
                // update row start + lane, from row 0 of token tb
                const uint32_t bo = upd_off(phase + lane, p.nh, p.inv_nh, (int)p.bst, (int)p.bstu);
                if (p.beta16) {
                    if (lane < len) pre.blogit = bf2f(p.beta16[(int64_t)tb * p.bst + bo + h]);
                } else {
                    const uint32_t nrec = __builtin_amdgcn_readfirstlane(
                        4u * (upd_off(phase + len - 1, p.nh, p.inv_nh, (int)p.bst, (int)p.bstu) + 1));
                    const i32x4 rb = make_rsrc(p.beta + (int64_t)tb * p.bst + h, nrec);
                    b2l_dword(rb, s_b, lane < len ? 4u * bo : nrec);
                }
            }
        }
    };
    if ((int)blockIdx.x < items) {
        const Item first = item_info(blockIdx.x);
        issue_k(first);
        issue_qgb(first);
    }
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const Item item = item_info(it);
        const int ci = item.ci, h = item.h, hk = item.hk, start = item.start, len = item.len;
        const int64_t ch_h = (int64_t)ci * p.HV + h;
        // The lane index for the lane masks of this item (the scan, the diagonal of G and
        // the causal masks of A, P^T and T) goes through an empty asm, so that the compiler
        // forms those masks where they are used instead of hoisting all of them out of the
        // item loop, where they do not fit in the scalar registers and are spilled.
        int lm = lane;
        asm volatile("" : "+v"(lm));
        const int cm = lm & 31, hm = lm >> 5;

        // ---- 1: q, g, beta (and k) were issued one item ahead
        const int tb = GDP ? __builtin_amdgcn_readfirstlane(start / p.nh) : start;
        const int phase = start - tb * p.nh;
        const float blogit = pre.blogit, graw = pre.graw;
        const bool gfirst = pre.gfirst;
        vm_wait<0>();
        lds_barrier();

        // ---- 2a: r_q and r_k from the q and k rows (16 rows per wave, 4 lanes per row)
        {
            const int row = 16 * wave + (lane >> 2);
            auto rnorm = [&](const lds_u32x4 *tile) {
                float s2 = 0.f;
#pragma unroll
                for (int i = 0; i < PK / 4; ++i)
                    s2 += sumsq8(__builtin_bit_cast(uint4, lds_row8<PK>(tile, row, 8 * (4 * i + (lane & 3)))));
                s2 += xch1(s2);
                s2 += xch2(s2);
                return row < len ? (p.l2norm ? 1.0f / sqrtf(s2 + 1e-6f) : 1.0f) : 0.f;
            };
            if (FWD) {
                const float rq = rnorm(sX);
                if ((lane & 3) == 0) s_rq[row] = rq;
            }
            const float rk = rnorm(sK);
            if ((lane & 3) == 0) s_rk[row] = rk;
        }
        // ---- 2b: Gram tiles.  wave 0: G(0,0); wave 1: G(1,0); wave 2: G(1,1); P^T(0,0) on wave
        // 1 (the reverse pass's operand mode: wave 0), P^T(1,1) on wave 2, P^T(0,1) on wave 3,
        // which also scans the gate.  Tile (m, n): rows 32 m.., columns 32 n..  The forward's
        // P^T tiles are scaled and stored by waves 1..3 while wave 0 inverts T's diagonal blocks.
        f32x16 Gt = {}, Pt = {}, Pq = {};
        const int gm = wave == 0 ? 0 : 1, gn = wave == 2 ? 1 : 0;   // G tile of waves 0..2
        const int pw = BW ? 1 : 0;                                   // the wave without a P^T tile
        const int pm = wave == 2 ? 1 : 0, pn = wave < 2 ? 0 : 1;     // P^T tile of the others
        if (wave < 3) {
#pragma unroll
            for (int s = 0; s < K / 16; ++s)
                Gt = mfma32(lds_row8<PK>(sK, 32 * gm + c, 16 * s + 8 * hh), lds_row8<PK>(sK, 32 * gn + c, 16 * s + 8 * hh), Gt);
        }
        if (FWD && WANT_V && wave != pw) {
#pragma unroll
            for (int s = 0; s < K / 16; ++s)
                Pt = mfma32(lds_row8<PK>(sK, 32 * pm + c, 16 * s + 8 * hh), lds_row8<PK>(sX, 32 * pn + c, 16 * s + 8 * hh), Pt);
        }
        if (BW && wave != 1) {
            // the same tile transposed, P = Q K^T (rows tokens t, columns s): its registers
            // 8 js .. 8 js + 7 are the A operand of P^T (lane s, tokens t in accumulator order)
#pragma unroll
            for (int s = 0; s < K / 16; ++s)
                Pq = mfma32(lds_row8<PK>(sX, 32 * pn + c, 16 * s + 8 * hh), lds_row8<PK>(sK, 32 * pm + c, 16 * s + 8 * hh), Pq);
        }
        if (wave == 3) {
            // the gate and beta transforms fused into the prologue (the cudnn-frontend PR
            // "Further reduce FROST LA CPU overhead + fully support all L2norm, beta, gate
            // fusion", commit notes: safe_gate with a_log / dt_bias, use_beta_sigmoid_in_kernel)
            float gr = GDP ? graw : s_g[lane];
            if (p.a_log) {
                const float x = gr + (p.dt_bias ? p.dt_bias[h] : 0.f);
                const float softplus = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
                gr = (lane < len && gfirst) ? -expf(p.a_log[h]) * softplus : 0.f;
            }
            if (p.beta16) s_b[lane] = lane < len ? 1.f / (1.f + expf(-blogit)) : 0.f;
            // inclusive scan of g log2(e) (zeros past the end)
            float xg = gr * kLog2e;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(xg, off, 64);
                if (lm >= off) xg += y;
            }
            s_gam[lane] = xg;
        }
        lds_barrier();

        // ---- 2c: v into q's space (every q read is done); per-token factors and the inter
        // pass's scalars; A^T (waves 0..2); the reverse pass's operand mode's P^T out
        if (!WANT_V) {
        } else if (!GDP)
            intra_load_tile<V>(sX, p.v + (int64_t)start * p.vst + (int64_t)h * p.vsh, 2u * (uint32_t)p.vst, len,
                               wave, lane, 4);
        else
            intra_load_urows<V>(sX, p.v + (int64_t)tb * p.vst + (int64_t)h * p.vsh, (int)p.vst, (int)p.vstu, phase,
                                len, p.nh, p.inv_nh, wave, lane, 4);
        const float gl = s_gam[len - 1];
        // the per-token factors and the inter pass's scalars: wave 3 in the forward (free
        // here: its P^T tile is stored later), wave 1 in the reverse pass's operand mode
        if (wave == (BW ? 1 : 3)) {
            const int t = lane;
            const float gm_t = s_gam[t], rk = s_rk[t];
            s_fw[t] = s_b[t] * exp2_hw(gm_t) * rk;
            float *sc = w.SC + ch_h * kScalars;
            sc[t] = exp2_hw(gl - gm_t) * rk;                                         // d (0 past the end)
            sc[64 + t] = (FWD && t < len) ? p.scale * s_rq[t] * exp2_hw(gm_t) : 0.f;   // sq
            if (t == 0) sc[192] = exp2_hw(gl);
            if (BW == 2) {
                // the backward's intra pass: gam (log2 units), r_k, r_q, beta per token
                float *sb = w.SB + ch_h * kScalars;
                sb[t] = gm_t;
                sb[64 + t] = rk;
                sb[128 + t] = s_rq[t];
                sb[192 + t] = s_b[t];
            }
        }
        if (wave < 3) {
            // A[t][s] for this lane's column s and rows t = 32 gm + 8 j + 4 hh + i, stored as A^T[s][t..]
            const int s = 32 * gn + c;
            const float gs = s_gam[s], rs = s_rk[s];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t0 = 32 * gm + 8 * j + 4 * hh;
                const f32x4 gt = *reinterpret_cast<const lds_f32x4 *>(s_gam + t0);
                const f32x4 rt = *reinterpret_cast<const lds_f32x4 *>(s_rk + t0);
                const f32x4 bt = *reinterpret_cast<const lds_f32x4 *>(s_b + t0);
                f32x4 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = exp2_hw(32 * gn + cm < 32 * gm + 8 * j + 4 * hm + i ? gt[i] - gs : kNegInf);
                    a[i] = bt[i] * rt[i] * rs * e * Gt[4 * j + i];
                }
                *reinterpret_cast<lds_f32x4 *>(sAT + s * TS + t0) = a;
            }
        }
        if (BW && wave != 1) {
            // P tile (t tile pn, s tile pm): lane (c, hh) holds column s = 32 pm + c, rows
            // t = 32 pn + 8 j + 4 hh + i; written as the A fragments of P^T, [s tile + t tile][js]
            const int sI = 32 * pm + c;
            const float gs = s_gam[sI], rs = s_rk[sI] * p.scale;
            f32x16 pv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t0 = 32 * pn + 8 * j + 4 * hh;
                const f32x4 gt = *reinterpret_cast<const lds_f32x4 *>(s_gam + t0);
                const f32x4 rq = *reinterpret_cast<const lds_f32x4 *>(s_rq + t0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = exp2_hw(32 * pm + cm <= 32 * pn + 8 * j + 4 * hm + i ? gt[i] - gs : kNegInf);
                    pv[4 * j + i] = rq[i] * rs * e * Pq[4 * j + i];
                }
            }
#pragma unroll
            for (int js = 0; js < 2; ++js)
                w.PTF[(ch_h * 6 + 2 * (pm + pn) + js) * 64 + lane] = __builtin_bit_cast(uint4, pack32(pv, js));
        }
        // P^T tile (pm, pn) scaled, masked and stored: lane (c, hh) holds column t = 32 pn + c,
        // rows s = 32 pm + 8 j + 4 hh + i; registers 8 js .. 8 js + 7 are the B operand of token
        // tile pn, step 2 pm + js
        auto store_pt = [&]() {
            const int t = 32 * pn + c;
            const float gt = s_gam[t], rq = s_rq[t] * p.scale;
            f32x16 pv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s0 = 32 * pm + 8 * j + 4 * hh;
                const f32x4 gs = *reinterpret_cast<const lds_f32x4 *>(s_gam + s0);
                const f32x4 rs = *reinterpret_cast<const lds_f32x4 *>(s_rk + s0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = exp2_hw(32 * pm + 8 * j + 4 * hm + i <= 32 * pn + cm ? gt - gs[i] : kNegInf);
                    pv[4 * j + i] = rq * rs[i] * e * Pt[4 * j + i];
                }
            }
#pragma unroll
            for (int js = 0; js < 2; ++js) {
                const int f = (pn == 0 ? 0 : 2) + 2 * pm + js;
                st_op<NT>(reinterpret_cast<u32x4 *>(&w.PF[(ch_h * 6 + f) * 64 + lane]), __builtin_bit_cast(u32x4, pack32(pv, js)));
            }
        };
        if (BW && FWD && WANT_V && wave != pw) store_pt();
        lds_barrier();

        // ---- 3a: diagonal blocks D_b = (I + A_bb)^-1 (wave 0; lane 16 b + cc holds column cc of D_b)
        if (wave == 0) {
            const int b = lane >> 4, cc = lane & 15, o = 16 * b;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == (lm & 15)) ? 1.f : 0.f;
#pragma unroll
            for (int k = 0; k < 15; ++k) {
                // A[o + i][o + k] for i > k is A^T[o + k][o + i]: the row in four 16-byte
                // reads (independent of x, so they can be issued ahead of the chain)
                const lds_f32x4 *ar = reinterpret_cast<const lds_f32x4 *>(sAT + (o + k) * TS + o);
                float a[16];
#pragma unroll
                for (int q = (k + 1) / 4; q < 4; ++q) {
                    const f32x4 v = ar[q];
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[4 * q + e] = v[e];
                }
                const float xk = x[k];
#pragma unroll
                for (int i = k + 1; i < 16; ++i) x[i] = fmaf(-a[i], xk, x[i]);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sAT[(o + i) * TS + o + cc] = x[i];
        } else if (!BW && FWD && WANT_V) {
            store_pt();
        }
        lds_barrier();

        // ---- 3b: block rows 1..3.  Block (i, j), wave (i - 1 - j): R = sum_k A_ik T_kj, then
        // T_ij = -D_i R with R's rows taken in accumulator order (lane (col cc, quad q) holds
        // R[4 q + e][cc] in register e, which step e of the product reads as row 4 q + e).
        {
            const int cc = lane & 15, q = lane >> 4;
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                const int j = i - 1 - wave;
                if (j >= 0) {
                    f32x4 R = {0.f, 0.f, 0.f, 0.f};
                    for (int k = j; k < i; ++k) {
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            // A_ik[cc][4 s + q] = A^T[16 k + 4 s + q][16 i + cc];  T_kj[4 s + q][cc]
                            const float a = sAT[(16 * k + 4 * s + q) * TS + 16 * i + cc];
                            const float t = sAT[(16 * k + 4 * s + q) * TS + 16 * j + cc];
                            R = mfma_f32(a, t, R);
                        }
                    }
                    f32x4 Tij = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        // -D_i[cc][4 q + s] pairs with R[4 q + s][.] held in register s
                        const float dneg = -sAT[(16 * i + cc) * TS + 16 * i + 4 * q + s];
                        Tij = mfma_f32(dneg, R[s], Tij);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) sAT[(16 * i + 4 * q + e) * TS + 16 * j + cc] = Tij[e];
                }
                // The A^T blocks of finished block rows are dead: the idle wave zeroes them
                // (block (0, 1) once row 1 is done, (0, 2) and (1, 2) once row 2 is), so that
                // above the diagonal T reads as zero in step 4 except in block column 3.
                if (i >= 2 && wave == i) {
                    const int zr = lane >> 2, zc = 4 * (lane & 3);
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    for (int k = 0; k < i - 1; ++k)
                        *reinterpret_cast<lds_f32x4 *>(sAT + (16 * k + zr) * TS + 16 * (i - 1) + zc) = z;
                }
                if (i == 3) vm_wait<0>();   // v (this wave's share), before the last barrier
                lds_barrier();
            }
        }

        if (BW == 2) {
            // T (unit lower triangular) in bf16, row-major 64 x 64, for the backward's intra pass
            const int row = tid >> 2, c0 = 16 * (tid & 3);
            bf16x8 tv[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) tv[e >> 3][e & 7] = f2bf(c0 + e <= row ? sAT[row * TS + c0 + e] : 0.f);
            uint4 *dst = w.TB + ch_h * (64 * 64 / 8) + row * 8 + 2 * (tid & 3);
            dst[0] = __builtin_bit_cast(uint4, tv[0]);
            dst[1] = __builtin_bit_cast(uint4, tv[1]);
        }

        // ---- 4: -W (W^T = K^T Tw^T: rows key columns, columns tokens; registers 8 js ..
        // 8 js + 7 are the A operand rows of W for one reduction step) and U~ = Thi V + Tlo V,
        // with Tw = T diag(beta 2^gam r_k) and T diag(beta) = Thi + Tlo (bf16) formed in
        // registers: wave w only needs rows 32 m .. 32 m + 31 of them, m = w & 1, and both
        // products read them at (row 32 m + c, columns 16 s + 8 hh .. + 7).  T is zero above
        // the diagonal (the array holds A^T there).
        {
            const int m = wave & 1, t = 32 * m + c;
            // Above the diagonal the array holds zeros (the diagonal blocks from 3a, blocks
            // (0, 1), (0, 2), (1, 2) from 3b) except for block column 3 of rows 0 .. 47, which
            // still holds A^T: masked here by the row.
            const bool col3 = 32 * m + cm >= 48;
            // T[t][16 s + 8 hh + e] (zero above the diagonal), times the per-column factor f
            auto trow = [&](int s, const lds_float *f, float (&o)[8]) {
                const int s0 = 16 * s + 8 * hh;
                const f32x4 t0 = *reinterpret_cast<const lds_f32x4 *>(sAT + t * TS + s0);
                const f32x4 t1 = *reinterpret_cast<const lds_f32x4 *>(sAT + t * TS + s0 + 4);
                const f32x4 f0 = *reinterpret_cast<const lds_f32x4 *>(f + s0);
                const f32x4 f1 = *reinterpret_cast<const lds_f32x4 *>(f + s0 + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[e] = (s < 3 || col3) ? (e < 4 ? t0[e] * f0[e] : t1[e - 4] * f1[e - 4]) : 0.f;
            };
            {
                bf16x8 tw[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    float o[8];
                    trow(s, s_fw, o);
#pragma unroll
                    for (int e = 0; e < 8; ++e) tw[s][e] = f2bf(o[e]);
                }
#pragma unroll
                for (int i = 0; i < (2 * (K / 32)) / 4; ++i) {
                    const int nb = 2 * i + (wave >> 1);
                    if (WANT_V) {
                        f32x16 acc = {};
#pragma unroll
                        for (int s = 0; s < 4; ++s) acc = mfma32(lds_tr32s<PK, false>(sK, 16 * s, 32 * nb, lane), tw[s], acc);
#pragma unroll
                        for (int js = 0; js < 2; ++js) {
                            const int kg = 2 * nb + js, kh = kg / NKS, kk = kg % NKS;
                            st_op<NT>(reinterpret_cast<u32x4 *>(&w.WF[(ch_h * (K / 8) + (kh * 2 + m) * NKS + kk) * 64 + lane]),
                                  __builtin_bit_cast(u32x4, neg_bf16(pack32(acc, js))));
                        }
                    }
                    if (BW) {
                        // W = Tw K itself (operands swapped): rows tokens of tile m in accumulator
                        // order, lane = key column, so registers 8 js .. 8 js + 7 are the A operand
                        // of W^T for token step 2 m + js; written negated, [key tile][token step]
                        f32x16 acc = {};
#pragma unroll
                        for (int s = 0; s < 4; ++s) acc = mfma32(tw[s], lds_tr32s<PK, false>(sK, 16 * s, 32 * nb, lane), acc);
#pragma unroll
                        for (int js = 0; js < 2; ++js)
                            w.WTF[((ch_h * (K / 32) + nb) * 4 + 2 * m + js) * 64 + lane] = neg_bf16(pack32(acc, js));
                    }
                }
            }
            // every wave is done with sK: the next item's k rows go there now
            lds_barrier();
            const bool more = it + (int)gridDim.x < items;
            const Item nxt = item_info(more ? it + gridDim.x : it);
            if (more) issue_k(nxt);
            if (!WANT_V) {
                if (more) issue_qgb(nxt);   // sX and the scalars are done with too
                continue;
            }
            // hi = bf16(x) two at a time (one conversion per pair), read back by a shift or a
            // mask; lo = bf16(x - hi), x - hi being exact
            bf16x8 th[4], tl[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float o[8];
                trow(s, s_b, o);
                u32x4 hv, lv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t hp = __builtin_bit_cast(uint32_t, bf16x2{f2bf(o[2 * e]), f2bf(o[2 * e + 1])});
                    asm volatile("" : "+v"(hp));   // the low half by a shift, not a second conversion
                    const float h0 = __uint_as_float(hp << 16), h1 = __uint_as_float(hp & 0xffff0000u);
                    hv[e] = hp;
                    lv[e] = __builtin_bit_cast(uint32_t, bf16x2{f2bf(o[2 * e] - h0), f2bf(o[2 * e + 1] - h1)});
                }
                th[s] = __builtin_bit_cast(bf16x8, hv);
                tl[s] = __builtin_bit_cast(bf16x8, lv);
            }
            constexpr int NU = (2 * (V / 32)) / 4;
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                const int ct = 2 * i + (wave >> 1);
                f32x16 acc = {};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 vb = lds_tr32s<PV, false>(sX, 16 * s, 32 * ct, lane);
                    acc = mfma32(th[s], vb, acc);
                    acc = mfma32(tl[s], vb, acc);
                }
                if (i == NU - 1) {
                    // every wave is done with sX (v) and the scalars: the next item's q, g
                    // and beta go there now, under this item's last stores
                    lds_barrier();
                    if (more) issue_qgb(nxt);
                }
                const int sh = f16_tile_shift(acc);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    st_op<NT>(reinterpret_cast<u32x2 *>(&w.UH[(((ch_h * (V / 32) + ct) * 2 + m) * 4 + j) * 64 + lane]),
                          __builtin_bit_cast(u32x2, f16_pack4(acc, j, sh)));
                if (lane == 0) w.SC[ch_h * kScalars + 128 + 2 * ct + m] = __int_as_float(sh);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_inter: one workgroup of 6 waves per (sequence, value head, 32 state columns),
// on 32 x 32 MFMA tiles, with three roles:
//   state waves kh = 0, 1 (waves 0, 1) own the state rows of key half kh (K/2 x 32
//     as accumulator tiles) and carry the chunk recurrence;
//   output waves t = 0, 1 (waves 2, 3) produce the outputs of 32-token tile t;
//   loader waves (waves 4, 5) issue every load of the chunk operands into LDS.
// Per chunk, with S the chunk's start state:
//   state wave kh:  X_kh = U~_kh + (-W)_kh S_kh  (its half of the reduction; U~
//                   rows of token tile kh, zero elsewhere); the X partials are swapped through LDS so that
//                   both hold U_new = X_0 + X_1 (fp32 addition commutes: the same
//                   bits in both); S_kh <- 2^(gam_n) S_kh + K_kh^T (diag(d) U_new),
//                   d = 2^(gam_n - gam) r_k, with K^T read from the raw k rows by
//                   LDS transpose reads.  It also publishes S (bf16) and its token
//                   tile of U_new (bf16) for the output waves.
//   output wave t:  Y^T = S^T Q_t^T over all state rows (after the first barrier),
//                   then at the start of the next chunk
//                   O^T = diag(sq) Y^T + U_new^T P_t^T, sq = scale r_q 2^gam
//                   (P causal: tile 0 needs U_new rows 0..31 only), and stores it.
// The reduction index of every product over state rows or tokens is in
// accumulator order, so S and U_new go from accumulators to operands in
// registers; the intra-chunk pass writes -W, P^T and U~ in that order.  Two barriers
// per chunk: B1 after the X partials and S are published, B2 at the end of the
// chunk.
//
// Loads: -W and U~ are stored in fragment order, so each state wave loads its own
// straight into registers (one coalesced 1 KiB load per fragment), two chunks
// ahead, into two register sets used by alternate chunks (U~ one chunk ahead).
// The loader waves keep the LDS operands in rotating buffers: raw k in two (read
// by the state waves at the start of chunk c, so right after B1 of chunk c the
// loaders issue the k rows of chunk c + 2 into the same buffer) and raw q, P^T and
// the scalars in three (those of chunk c + 2 are issued at the start of chunk c);
// before B2 of chunk c they wait for all of chunk c + 1's.  The k loads have one
// and a half chunk steps to land, the others two.  The loader loads are buffer
// loads into LDS written as asm:
// the compiler neither tracks them nor adds waits for them; the loader waves issue
// nothing else, so each wait counts exactly the loads issued after the ones it
// needs (loads complete in issue order).  Rows of k and q past a chunk's end are
// out of the buffer's range and load as zeros.  The barriers order LDS only.
// For the summary (k_inter_sum) the state is widened to [S | P] (K x (V + K)): the
// P columns start at the identity and see U~ = 0, so they evolve as the product of
// the decayed erase steps; there are no outputs and no output waves (the loader
// waves are waves 2, 3).

template <int K, int V, bool SUMMARY, int TP = 1, bool NOOUT = false>
struct InterCfg {
    static constexpr bool FWD = !SUMMARY;
    static constexpr bool OUT = FWD && !NOOUT;    // output waves and their operands (q, P^T)
    static constexpr int VA = SUMMARY ? V + K : V;
    static constexpr int NT = VA / (32 * TP);     // workgroups (TP 32-column tiles each) per (sequence, head)
    static constexpr int KH = K / 2;              // state rows per state wave
    static constexpr int NR = KH / 32;            // 32-row accumulator tiles per state wave
    static constexpr int NKS = KH / 16;           // reduction steps over a key half
    static constexpr int PPR = K / 8;             // 16-byte pieces per k or q row
    // operands in the workspace, per (chunk, head), in 1 KiB fragments: -W
    // [kh][token tile][step] (FW), loaded by the state waves straight into registers, and
    // U~ [value tile][token tile][j] in fp16 (FU per value tile).  In LDS: U~, raw k (64 x K
    // bf16, pieces swizzled by row) in its own array; raw q (same layout), P^T (tile
    // 0 steps 0..1, tile 1 steps 0..3) and the scalars (d[64], sq[64], 2^(gam_n) at
    // 192) in the other.
    static constexpr int FW = 4 * NKS, FU = 4 * TP, FQ = OUT ? K / 8 : 0, FP = OUT ? 6 : 0, FS = 1;
    static constexpr int oU = 0, oQ = oU + FU, oP = oQ + FQ, oS = oP + FP, NFE = oS + FS;
    static constexpr int FK = K / 8, oK = 0, NFL = FK;
    static constexpr int NKL = FK / 2;            // k tile loads per loader wave
    // waves: 0 .. 2 TP - 1 state (key half w & 1, tile w >> 1), (forward) two output waves,
    // then the two loader waves; the summary has no outputs, so its workgroup is 4 waves and
    // two fit on a CU
    static constexpr int SW = 2 * TP;             // state waves
    static constexpr int LW = OUT ? SW + 2 : SW;  // first loader wave
    static constexpr int THREADS = 64 * (LW + 2);
    static constexpr int NQ = NKL;                // q tile loads per loader wave (forward)
};

template <int K, int V, bool SUMMARY>
struct InterCtx {
    int nch, seq_start, seq_len, cid0, h, hk, tile, lane;
    int vt0;          // the workgroup's first 32-column value tile
    bool ptile;
};

// Loader wave lh, its half of chunk ci's raw k rows into `lb`.  Returns the
// number of loads.
// Gated Delta Product: where a chunk of update rows starts, token tb and update `phase`
// of it (uniform).  A sequence starts at a token's first update; each chunk is 64 updates
// on, so the loaders step the cursor instead of dividing by nh per chunk.
struct UCursor {
    int tb, phase;
    __device__ void advance(int q64, int r64, int nh)   // q64 = 64 / nh, r64 = 64 % nh
    {
        tb += q64;
        phase += r64;
        if (phase >= nh) { phase -= nh; ++tb; }
    }
};

// Gated Delta Product: koff holds the offsets of the pieces' rows for a chunk that starts at
// its token's first update (row = a nh + b: a tokens and b updates on), kb the b of each row.
template <int K, int V, bool SUMMARY, bool GDP>
__device__ __forceinline__ int inter_issue_k(const Prob &p, lds_u32x4 *lb, int ci, int lh,
                                             const InterCtx<K, V, SUMMARY> &x,
                                             const uint32_t (&koff)[InterCfg<K, V, SUMMARY>::NKL],
                                             const int (&kb)[InterCfg<K, V, SUMMARY>::NKL], UCursor cur)
{
    using C = InterCfg<K, V, SUMMARY>;
    const int start = x.seq_start + kChunk * ci, len = min(kChunk, x.seq_len - kChunk * ci);
    if (!GDP) {
        const i32x4 rK = make_rsrc(p.k + (int64_t)start * p.kst + (int64_t)x.hk * p.ksh,
                                   (uint32_t)len * 2u * (uint32_t)p.kst);
#pragma unroll
        for (int i = 0; i < C::NKL; ++i) b2l(rK, lb, C::oK + 2 * i + lh, koff[i], 0);
    } else {
        // Gated Delta Product: the chunk starts `phase` updates into token tb, so row a nh + b
        // is a tokens and b + phase updates on, or a + 1 tokens and b + phase - nh updates
        // once b + phase >= nh.  Offsets grow with the row (the token stride covers a token's
        // updates), so rows past the end lie past the range and load as zeros.
        const int tb = __builtin_amdgcn_readfirstlane(cur.tb), phase = __builtin_amdgcn_readfirstlane(cur.phase);
        const int st = (int)p.kst, su = (int)p.kstu;
        // the last row: lt tokens and phase + len - 1 - lt nh updates on (a quotient below 128)
        const int lt = __builtin_amdgcn_readfirstlane((int)(((float)(phase + len - 1) + 0.5f) * p.inv_nh));
        const uint32_t nrec = __builtin_amdgcn_readfirstlane(2u * (uint32_t)(lt * st + (phase + len - 1 - lt * p.nh) * su + K));
        const i32x4 rK = make_rsrc(p.k + (int64_t)tb * p.kst + (int64_t)x.hk * p.ksh, nrec);
        const uint32_t u0 = 2u * (uint32_t)(phase * su), u1 = u0 + 2u * (uint32_t)(st - p.nh * su);
        const int thr = p.nh - phase;
#pragma unroll
        for (int i = 0; i < C::NKL; ++i) b2l(rK, lb, C::oK + 2 * i + lh, koff[i] + (kb[i] >= thr ? u1 : u0), 0);
    }
    return C::NKL;
}

// Loader wave lh, its half of chunk ci's output operands (raw q, P^T) and the
// scalars (loader 0) into `eb`.  Returns the number of loads.
// Gated Delta Product: qoff holds the token offsets of the pieces' rows (a of row = a nh + b)
// for a chunk that starts at its token's first update, kb the b and krow the row of each.
template <int K, int V, bool SUMMARY, bool GDP, bool NOOUT = false, int TP = 1>
__device__ __forceinline__ int inter_issue_output(const Prob &p, const Ws &w, lds_u32x4 *eb, int ci, int lh,
                                                  const InterCtx<K, V, SUMMARY> &x,
                                                  const uint32_t (&qoff)[InterCfg<K, V, SUMMARY>::NQ],
                                                  const int (&kb)[InterCfg<K, V, SUMMARY>::NKL],
                                                  const int (&krow)[InterCfg<K, V, SUMMARY>::NKL], UCursor cur)
{
    using C = InterCfg<K, V, SUMMARY, TP, NOOUT>;
    const int64_t chh = (int64_t)(x.cid0 + ci) * p.HV + x.h;
    const uint32_t lo16 = (uint32_t)x.lane * 16u;
    int n = 0;
    if (C::OUT) {
        const int start = x.seq_start + kChunk * ci, len = min(kChunk, x.seq_len - kChunk * ci);
        if (!GDP) {
            const i32x4 rQ = make_rsrc(p.q + (int64_t)start * p.qst + (int64_t)x.hk * p.qsh,
                                       (uint32_t)len * 2u * (uint32_t)p.qst);
#pragma unroll
            for (int i = 0; i < C::FQ / 2; ++i) b2l(rQ, eb, C::oQ + 2 * i + lh, qoff[i], 0);
        } else {
            // Gated Delta Product: update row start + row reads q row (start + row) / nh at its
            // token's last update, zeros otherwise (offset past the buffer's range).  Row
            // a nh + b is update b + phase of token tb + a, or, once b + phase >= nh, update
            // b + phase - nh of token tb + a + 1.
            const int tb = __builtin_amdgcn_readfirstlane(cur.tb), phase = __builtin_amdgcn_readfirstlane(cur.phase);
            const int thr = p.nh - phase;
            const uint32_t rs = 2u * (uint32_t)p.qst, nrec = gdp_q_range(p, tb);
            const i32x4 rQ = make_rsrc(p.q + (int64_t)tb * p.qst + (int64_t)x.hk * p.qsh, nrec);
#pragma unroll
            for (int i = 0; i < C::FQ / 2; ++i) {
                const bool wrap = kb[i] >= thr;
                const bool last = krow[i] < len && kb[i] + phase - (wrap ? p.nh : 0) == p.nh - 1;
                b2l(rQ, eb, C::oQ + 2 * i + lh, last ? qoff[i] + (wrap ? rs : 0u) : nrec, 0);
            }
        }
        const i32x4 rP = make_rsrc(reinterpret_cast<const char *>(w.PF) + chh * 6 * kFrag, 6 * kFrag);
#pragma unroll
        for (int i = 0; i < 3; ++i) b2l(rP, eb, C::oP + 3 * lh + i, lo16, (3 * lh + i) * kFrag);
        n += C::FQ / 2 + 3;
    }
    if (!x.ptile) {
        const i32x4 rU = make_rsrc(reinterpret_cast<const char *>(w.UH) + (chh * (V / 32) + x.vt0) * 4 * kFrag,
                                   C::FU * kFrag);
#pragma unroll
        for (int i = 0; i < C::FU / 2; ++i) {
            const int f = lh * (C::FU / 2) + i;
            b2l(rU, eb, C::oU + f, lo16, f * kFrag);
        }
        n += C::FU / 2;
    }
    if (lh == 0) {
        const i32x4 rS = make_rsrc(w.SC + chh * kScalars, kScalars * 4);
        b2l(rS, eb, C::oS, lo16, 0);
        n += 1;
    }
    return n;
}

// Output wave t: O^T of its token tile of the chunk whose Y^T it holds, stored
// to o.  Lane (c, hh) holds value columns 8 j + 4 hh .. + 3 of token 32 t + c.
// One output tile, computed and held until its store (so that the store can be issued
// away from the loaders' operand loads).
struct OutTile {
    uint2 v[4];
    __bf16 *ob;       // row start of this lane's 8-column group, or null (no row)
};

template <int K, int V, bool SUMMARY, bool GDP>
__device__ __forceinline__ OutTile inter_output(const Prob &p, const lds_u32x4 *xU, const f32x16 &Y, const bf16x8 (&Pf)[4],
                                                float sq, int t, int o_start, int o_len, const InterCtx<K, V, SUMMARY> &x,
                                                int vt)
{
    const int lane = x.lane, c = lane & 31, hh = lane >> 5;
    f32x16 O;
#pragma unroll
    for (int e = 0; e < 16; ++e) O[e] = sq * Y[e];
    O = mfma32(__builtin_bit_cast(bf16x8, xU[0 * 64 + lane]), Pf[0], O);
    O = mfma32(__builtin_bit_cast(bf16x8, xU[1 * 64 + lane]), Pf[1], O);
    if (t != 0) {
        O = mfma32(__builtin_bit_cast(bf16x8, xU[2 * 64 + lane]), Pf[2], O);
        O = mfma32(__builtin_bit_cast(bf16x8, xU[3 * 64 + lane]), Pf[3], O);
    }
    const int tok = 32 * t + c;
    // o row: the token itself, or (Gated Delta Product) the token whose last update it is
    const int u = o_start + tok;
    int orow = -1;
    if (tok < o_len) {
        if (!GDP) orow = u;
        else if (u % p.nh == p.nh - 1) orow = u / p.nh;
    }
    OutTile r;
    r.ob = orow >= 0 ? p.o + (int64_t)orow * p.ost + (int64_t)x.h * p.osh + 32 * vt + 4 * hh : nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 o4 = {O[4 * j], O[4 * j + 1], O[4 * j + 2], O[4 * j + 3]};
        const uint4 w4 = __builtin_bit_cast(uint4, pack_b(o4, o4));
        r.v[j] = make_uint2(w4.x, w4.y);
    }
    return r;
}

__device__ __forceinline__ void store_out(const OutTile &r)
{
    if (r.ob) {
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<uint2 *>(r.ob + 8 * j) = r.v[j];
    }
}

// Workgroup b of a chunk pass -> (sequence, value head, 32-column tile).  Blocks go in
// groups of 8 (sequence, q/k head) units x G value heads x NT tiles: consecutive blocks go
// to different XCDs, and the G NT workgroups of one (sequence, q/k head), which read the
// same k and q rows (and, per value head, the same -W), to the same XCD, where they are
// dispatched together and share its L2.  Units start longest sequence first.
struct UnitOfBlock {
    int n, h, tile;
};
__device__ __forceinline__ UnitOfBlock unit_of_block(const Prob &p, const Ws &w, int b, int NT)
{
    const int G = p.HV / p.HK, per = G * NT, UK = p.N * p.HK;
    const int grp = b / (8 * per), rem = b % (8 * per);
    const int ug = min(8, UK - 8 * grp);
    const int uk = 8 * grp + rem % ug, inner = rem / ug;
    UnitOfBlock r;
    r.tile = inner % NT;
    r.n = w.order[uk / p.HK];
    r.h = (uk % p.HK) * G + inner / NT;
    return r;
}

// NOOUT (with CK, fp32 rows): the states only, no outputs (the backward's run of the forward):
// no output waves (the loaders are waves 2, 3, as in the summary) and no q or P^T.
// TP = 2 (the plain forward at large batch): two 32-column tiles per workgroup, so that a
// batch needs half the workgroups, with four state waves (key half x tile), the output waves
// covering both tiles, and the output operands double- instead of triple-buffered (LDS).
template <int K, int V, bool SUMMARY, bool CK = false, bool GDP = false, bool NOOUT = false, int TP = 1>
__device__ __forceinline__ void inter_body(const Prob &p, const Ws &w)
{
    static_assert(!NOOUT || (CK && !SUMMARY && !GDP), "states only: the forward with the fp32 series");
    static_assert(TP == 1 || !GDP, "two tiles per workgroup: not the Gated Delta Product");
    using C = InterCfg<K, V, SUMMARY, TP, NOOUT>;
    constexpr int NR = C::NR, NKS = C::NKS;
    constexpr int NEB = TP == 1 ? 3 : 2;                   // output-operand buffers
    __shared__ u32x4 sE0[C::NFE * 64], sE1[C::NFE * 64], sE2[NEB == 3 ? C::NFE * 64 : 1];   // q, U~, P^T, scalars
    __shared__ u32x4 sL0[C::NFL * 64], sL1[C::NFL * 64];   // raw k: two buffers
    __shared__ u32x4 sX[TP * 2 * 8 * 64];                  // X partials: [tile][kh][m][j][lane]
    __shared__ u32x4 sS[C::OUT ? TP * 2 * NKS * 64 : 1];   // S (bf16 operands): [tile][kh][step][lane]
    __shared__ u32x4 sU[C::OUT ? TP * 4 * 64 : 1];         // U_new (bf16 operands): [tile][token step][lane]
    lds_u32x4 *const e0 = (lds_u32x4 *)sE0, *const e1 = (lds_u32x4 *)sE1, *const e2 = (lds_u32x4 *)sE2;
    auto ebuf = [&](int c) {
        if (NEB == 2) return (c & 1) ? e1 : e0;
        const int r = c % 3;
        return r == 0 ? e0 : (r == 1 ? e1 : e2);
    };
    lds_u32x4 *const l0 = (lds_u32x4 *)sL0, *const l1 = (lds_u32x4 *)sL1;

    if (w.hdr[0] != LA_DEVICE_OK) return;
    const UnitOfBlock ub = unit_of_block(p, w, blockIdx.x, C::NT);
    const int n = ub.n, h = ub.h, tile = ub.tile;
    const int4 si = w.seq_info[n];

    InterCtx<K, V, SUMMARY> x;
    x.seq_start = si.x;
    x.seq_len = si.y;
    x.cid0 = si.z;
    x.nch = (x.seq_len + kChunk - 1) / kChunk;
    x.h = h;
    x.hk = h / (p.HV / p.HK);
    x.tile = tile;
    x.vt0 = TP * tile;
    x.lane = threadIdx.x & 63;
    x.ptile = SUMMARY && 32 * x.vt0 >= V;   // the workgroup's tiles are all P columns or all S columns
    // Roles by wave: with two 4-wave workgroups per CU the hardware puts a workgroup's waves
    // 0..3 on SIMDs s, s + 2, s + 1, s + 3 of a fixed cycle and, for most CUs, the other
    // workgroup's one step further on, so in the states-only forward the state roles go to
    // hardware waves 0 and 2 (and the loaders to 1 and 3): the two workgroups' state waves
    // then sit on four different SIMDs instead of sharing one (dense batch: 612 -> 606 us with
    // the reverse pass).  The summary keeps waves 0 and 1 (the same remap measured 0-2 %
    // slower there).
    const int hwave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = NOOUT && TP == 1 ? ((hwave & 1) << 1) | (hwave >> 1) : hwave;
    const int lane = x.lane, c = lane & 31, hh = lane >> 5;
    const int nch = x.nch;

    // State series (forward only): the state at the start of every chunk whose first
    // token is a multiple of ck_every tokens into the sequence is entry ck_base + j of
    // the series, j = that multiple; ck_base counts the entries of the sequences before
    // this one (ceil(length / ck_every) each), summed across the wave.  bf16 rows are
    // written by the output waves from the bf16 copy of S they read anyway (off the
    // state waves' chain, whose next loop-head wait would otherwise cover the stores);
    // fp32 rows by the state waves.
    int64_t ck_base = 0;
    if (CK && wave < C::LW) {
        int64_t part = 0;
        for (int s = lane; s < n; s += 64) part += (p.cu[s + 1] - p.cu[s] + p.ck_every - 1) / p.ck_every;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
        ck_base = part;
    }

    if (wave >= C::LW) {
        // ------------------------------------------------------------ loader waves
        const int lh = wave - C::LW;
        // source offsets of this lane's 16-byte pieces of the k and q tiles (LDS piece
        // (row, j) holds source piece j ^ swz_mask(row) of the row)
        uint32_t qoff[C::NQ], koff[C::NKL];
        int kb[C::NKL], krow[C::NKL];
#pragma unroll
        for (int i = 0; i < C::NKL; ++i) {
            const int s = (2 * i + lh) * 64 + lane;
            const int row = s / C::PPR, pc = (s % C::PPR) ^ swz_mask<C::PPR>(row);
            krow[i] = row;
            if (!GDP) {
                kb[i] = 0;
                koff[i] = (uint32_t)row * 2u * (uint32_t)p.kst + 16u * (uint32_t)pc;
                if (C::OUT) qoff[i] = (uint32_t)row * 2u * (uint32_t)p.qst + 16u * (uint32_t)pc;
            } else {
                const int a = row / p.nh;
                kb[i] = row - a * p.nh;
                koff[i] = 2u * (uint32_t)(a * (int)p.kst + kb[i] * (int)p.kstu) + 16u * (uint32_t)pc;
                if (C::OUT) qoff[i] = (uint32_t)a * 2u * (uint32_t)p.qst + 16u * (uint32_t)pc;
            }
        }
        // Gated Delta Product: the cursor of the next chunk to issue (chunk 0 starts at the
        // sequence's first token; every chunk is 64 update rows)
        const int q64 = GDP ? 64 / p.nh : 0, r64 = GDP ? 64 - q64 * p.nh : 0;
        UCursor cur{GDP ? __builtin_amdgcn_readfirstlane(x.seq_start / p.nh) : 0, 0};
        // chunk c's k rows land in k buffer c % 2, its output operands in buffer c % 3.
        // At the start of chunk c (after B2 of chunk c - 1, when chunk c - 1's output
        // operands are dead) the output operands of chunk c + 2 are issued, after B1 of
        // chunk c (the state waves have read chunk c's k by then) its k rows; before B2
        // of chunk c the loaders wait for all of chunk c + 1's.
        int na = 0, nb = 0;
        if (NEB == 2) {
            // two output-operand buffers: chunk c + 1's are issued at the start of chunk c
            // (after B2 of chunk c - 1, when chunk c - 1's are dead), its k rows one chunk
            // earlier, after B1 of chunk c - 1; before B2 of chunk c the loaders wait for
            // all of chunk c + 1's
            if (nch > 0) {
                na = inter_issue_k<K, V, SUMMARY, GDP>(p, l0, 0, lh, x, koff, kb, cur);
                nb = inter_issue_output<K, V, SUMMARY, GDP, NOOUT, TP>(p, w, e0, 0, lh, x, qoff, kb, krow, cur);
                if (nch > 1) inter_issue_k<K, V, SUMMARY, GDP>(p, l1, 1, lh, x, koff, kb, cur);
                vm_wait_n(nch > 1 ? na : 0);                  // all of chunk 0
            }
            lds_barrier();
            for (int ci = 0; ci < nch; ++ci) {
                const bool more1 = ci + 1 < nch, more2 = ci + 2 < nch;
                if (more1)
                    inter_issue_output<K, V, SUMMARY, GDP, NOOUT, TP>(p, w, ebuf(ci + 1), ci + 1, lh, x, qoff, kb, krow, cur);
                lds_barrier();                                // B1
                if (more2) inter_issue_k<K, V, SUMMARY, GDP>(p, (ci & 1) ? l1 : l0, ci + 2, lh, x, koff, kb, cur);
                vm_wait_n(more2 ? na : 0);                    // all of chunk ci + 1
                lds_barrier();                                // B2
            }
            return;
        }
        if (nch > 0) {
            na = inter_issue_k<K, V, SUMMARY, GDP>(p, l0, 0, lh, x, koff, kb, cur);
            nb = inter_issue_output<K, V, SUMMARY, GDP, NOOUT, TP>(p, w, e0, 0, lh, x, qoff, kb, krow, cur);
            if (GDP) cur.advance(q64, r64, p.nh);
            if (nch > 1) {
                inter_issue_k<K, V, SUMMARY, GDP>(p, l1, 1, lh, x, koff, kb, cur);
                inter_issue_output<K, V, SUMMARY, GDP, NOOUT, TP>(p, w, e1, 1, lh, x, qoff, kb, krow, cur);
                if (GDP) cur.advance(q64, r64, p.nh);
            }
            vm_wait_n(nch > 1 ? na + nb : 0);                 // all of chunk 0
        }
        lds_barrier();
        for (int ci = 0; ci < nch; ++ci) {
            const bool more2 = ci + 2 < nch;
            if (more2) inter_issue_output<K, V, SUMMARY, GDP, NOOUT, TP>(p, w, ebuf(ci + 2), ci + 2, lh, x, qoff, kb, krow, cur);
            lds_barrier();                                    // B1
            if (more2) {
                inter_issue_k<K, V, SUMMARY, GDP>(p, (ci & 1) ? l1 : l0, ci + 2, lh, x, koff, kb, cur);
                if (GDP) cur.advance(q64, r64, p.nh);
            }
            vm_wait_n(more2 ? na + nb : 0);                   // all of chunk ci + 1
            lds_barrier();                                    // B2
        }
        return;
    }

    lds_u32x4 *const xX = (lds_u32x4 *)sX, *const xS = (lds_u32x4 *)sS, *const xU = (lds_u32x4 *)sU;
    if (C::OUT && wave >= C::SW) {
        // ------------------------------------------------------------ output waves
        const int t = wave - C::SW;
        f32x16 Y[TP] = {};
        bf16x8 Pf[4];
        float sq = 0.f;
        int o_start = 0, o_len = 0;
        // With two tiles per workgroup the output tiles are stored at the end of the step, away
        // from the loaders' operand loads issued at its start (dense batch: k_inter_wide 160 ->
        // 148 us); with one tile, where the step is shorter, right away (the varlen batch's
        // k_inter measured 34.3 -> 35.3 us the other way).
        constexpr bool LATE = TP > 1;
        OutTile ot[TP];
        lds_barrier();
        for (int ci = 0; ci < nch; ++ci) {
            const lds_u32x4 *eb = ebuf(ci);
            // the previous chunk's output (its U_new was published before the last B2)
            if (ci > 0) {
#pragma unroll
                for (int tp = 0; tp < TP; ++tp) {
                    ot[tp] = inter_output<K, V, SUMMARY, GDP>(p, xU + tp * 4 * 64, Y[tp], Pf, sq, t, o_start, o_len, x,
                                                              x.vt0 + tp);
                    if (!LATE) store_out(ot[tp]);
                }
            }
            lds_barrier();                                    // B1: S of chunk ci is published
            // operands of chunk ci (they stay in their buffer until the next chunk
            // starts): q as B operands over all state rows (accumulator order within
            // each 32-row tile), P^T of tile t, sq
            bf16x8 Qf[2 * NKS];
            {
                const lds_u32x2 *ew = reinterpret_cast<const lds_u32x2 *>(eb);
                const int row = 32 * t + c;
#pragma unroll
                for (int kk = 0; kk < 2 * NKS; ++kk) {
                    const int col = 16 * kk + 4 * hh;
                    const u32x2 a0 = ew[C::oQ * 128 + (swz<C::PPR>(row, col) >> 3)];
                    const u32x2 a1 = ew[C::oQ * 128 + (swz<C::PPR>(row, col + 8) >> 3)];
                    Qf[kk] = __builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    Pf[s] = (s < 2 || t != 0) ? __builtin_bit_cast(bf16x8, eb[(C::oP + (t != 0 ? 2 : 0) + s) * 64 + lane])
                                              : bf16x8{};
                sq = reinterpret_cast<const lds_float *>(eb + C::oS * 64)[64 + 32 * t + c];
            }
#pragma unroll
            for (int tp = 0; tp < TP; ++tp) {
                Y[tp] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < 2 * NKS; ++kk)
                    Y[tp] = mfma32(__builtin_bit_cast(bf16x8, xS[(tp * 2 * NKS + kk) * 64 + lane]), Qf[kk], Y[tp]);
            }
            if (CK && !p.ck_fp32 && (kChunk * ci) % p.ck_every == 0) {
                // the chunk-start state as bf16 rows: output wave t writes key steps
                // t NKS .. t NKS + NKS - 1; lane (c, hh) of step kk holds column c, keys
                // 16 kk + 4 hh + e (slots e) and 16 kk + 8 + 4 hh + e (slots 4 + e)
                const int64_t e = ck_base + (int64_t)kChunk * ci / p.ck_every;
                if (e < p.ck_cap) {
#pragma unroll
                    for (int tp = 0; tp < TP; ++tp) {
                        __bf16 *dst = static_cast<__bf16 *>(p.ck) + ((e * p.HV + x.h) * K) * V + 32 * (x.vt0 + tp) + c;
#pragma unroll
                        for (int i = 0; i < NKS; ++i) {
                            const int kk = t * NKS + i;
                            const bf16x8 sv = __builtin_bit_cast(bf16x8, xS[(tp * 2 * NKS + kk) * 64 + lane]);
#pragma unroll
                            for (int slot = 0; slot < 8; ++slot)
                                dst[(int64_t)(16 * kk + 8 * (slot >> 2) + 4 * hh + (slot & 3)) * V] = sv[slot];
                        }
                    }
                }
            }
            if (LATE && ci > 0) {
#pragma unroll
                for (int tp = 0; tp < TP; ++tp) store_out(ot[tp]);
            }
            o_start = x.seq_start + kChunk * ci;
            o_len = min(kChunk, x.seq_len - kChunk * ci);
            lds_barrier();                                    // B2: U_new of chunk ci is published
        }
        if (nch > 0) {
#pragma unroll
            for (int tp = 0; tp < TP; ++tp)
                store_out(inter_output<K, V, SUMMARY, GDP>(p, xU + tp * 4 * 64, Y[tp], Pf, sq, t, o_start, o_len, x,
                                                           x.vt0 + tp));
        }
        return;
    }

    // ---------------------------------------------------------------- state waves
    // (they carry the sequential chain: first claim on their SIMDs' issue slots)
    __builtin_amdgcn_s_setprio(3);
    const int kh = wave & 1, tp = wave >> 1;            // key half, tile of the workgroup
    const int vt = x.vt0 + tp;                          // this wave's 32-column value tile
    const int col = 32 * vt + c;                        // this lane's state column
    // this wave's tile's X partials, S and U_new operands
    lds_u32x4 *const tX = xX + tp * 2 * 8 * 64, *const tS = xS + tp * 2 * NKS * 64, *const tU = xU + tp * 4 * 64;
    const int row0 = kh * C::KH;                        // first state row of this wave
    // the lane's part of the K^T transpose-read addresses (the chunk's token step adds a
    // uniform 16 PPR t0), computed once instead of in every chunk step (about 50 fewer VALU
    // instructions per step on the chain and 12 fewer VGPRs; k_inter 34.2 -> 34.0 us at the
    // varlen workload, k_inter_sum 1427 -> 1413 us at the summary one).  The kernel with the
    // fp32 series measured 49.8 -> 51.5 us that way and keeps the per-step form.
    constexpr bool KTR = !CK;
    uint2 ktr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) ktr[r] = tr_lane_off<C::PPR>(row0 + 32 * r, lane);
    const int64_t unit = (int64_t)n * p.HV + h;
    f32x16 S[NR];
    if (!x.ptile) {
        if (p.s0) {
            const float *s0 = p.s0 + unit * K * V;
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    S[r][e] = s0[(int64_t)(row0 + 32 * r + 8 * (e >> 2) + 4 * hh + (e & 3)) * V + col];
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r) S[r] = f32x16{};
        }
    } else {
        const int pc = col - V;
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int e = 0; e < 16; ++e) S[r][e] = (row0 + 32 * r + 8 * (e >> 2) + 4 * hh + (e & 3) == pc) ? 1.f : 0.f;
    }
    // Token tiles in this wave's order: o = 0 is its own tile (kh), o = 1 the other one
    // (only addresses depend on kh, never a register selection).  -W and U~ are stored
    // in fragment order: this wave loads its -W straight into registers, two chunks
    // ahead into two register sets used by alternate chunks; U~ comes through LDS with
    // the output operands.
    struct StateOps {
        bf16x8 W[2][NKS];
    };
    auto load_w = [&](StateOps &R, int cj) {
        const int64_t chh = (int64_t)(x.cid0 + cj) * p.HV + x.h;
        const uint4 *wsrc = w.WF + chh * C::FW * 64 + lane;
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
            for (int kk = 0; kk < NKS; ++kk)
                R.W[o][kk] = __builtin_bit_cast(bf16x8, wsrc[((kh * 2 + (o ^ kh)) * NKS + kk) * 64]);
    };
    StateOps opA, opB;
    if (nch > 0) load_w(opA, 0);
    if (nch > 1) load_w(opB, 1);
    lds_barrier();
    auto chunk_step = [&](int ci, StateOps &R) {
        const lds_u32x4 *eb = ebuf(ci);
        const lds_u32x4 *lb = (ci & 1) ? l1 : l0;
        // (stored here, at the start of the step, not at the end of the previous one: stores
        // issued after this wave's -W loads would be waited for with them at the loop head)
        if (CK && p.ck_fp32 && (kChunk * ci) % p.ck_every == 0) {
            const int64_t e = ck_base + (int64_t)kChunk * ci / p.ck_every;
            if (e < p.ck_cap) {
                float *base = static_cast<float *>(p.ck) + ((e * p.HV + h) * K) * V;
                if (p.ck_quad) {
#pragma unroll
                    for (int r = 0; r < NR; ++r)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            *reinterpret_cast<f32x4 *>(base + quad_off(row0 + 32 * r + 8 * j + 4 * hh, col, V)) =
                                f32x4{S[r][4 * j], S[r][4 * j + 1], S[r][4 * j + 2], S[r][4 * j + 3]};
                } else {
#pragma unroll
                    for (int r = 0; r < NR; ++r)
#pragma unroll
                        for (int ee = 0; ee < 16; ++ee)
                            base[(int64_t)(row0 + 32 * r + 8 * (ee >> 2) + 4 * hh + (ee & 3)) * V + col] = S[r][ee];
                }
            }
        }
        // ---- K^T of this key half (A operands: state rows, tokens in accumulator order,
        // own token tile first), read from the raw k rows while the X products run
        bf16x8 Kf[NR][4];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int o = 0; o < 2; ++o)
#pragma unroll
                for (int js = 0; js < 2; ++js)
                    Kf[r][2 * o + js] =
                        KTR ? lds_tr32s_at(reinterpret_cast<const lds_char *>(lb + C::oK * 64) +
                                               16 * C::PPR * 16 * (2 * (o ^ kh) + js), ktr[r])
                            : lds_tr32s<C::PPR, true>(lb + C::oK * 64, 16 * (2 * (o ^ kh) + js), row0 + 32 * r, lane);
        // U~ enters through the accumulator of the wave whose token tile it is
        f32x16 X[2];
        X[1] = f32x16{};
        if (!x.ptile) {
            const lds_u32x2 *uh = reinterpret_cast<const lds_u32x2 *>(eb + C::oU * 64) + (tp * 2 + kh) * 4 * 64;
            const int sh = __float_as_int(reinterpret_cast<const lds_float *>(eb + C::oS * 64)[128 + 2 * vt + kh]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 u4 = f16_unpack4(uh[j * 64 + lane], sh);
#pragma unroll
                for (int e = 0; e < 4; ++e) X[0][4 * j + e] = u4[e];
            }
        } else {
            X[0] = f32x16{};
        }
        // ---- S as bf16 operands, published for the output waves
        bf16x8 Sb[NKS];
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
            Sb[kk] = pack32(S[kk >> 1], kk & 1);
            if (C::OUT) tS[(kh * NKS + kk) * 64 + lane] = __builtin_bit_cast(u32x4, Sb[kk]);
        }
        // ---- X_kh = [U~] + (-W)_kh S_kh, published for the other state wave
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk)
#pragma unroll
            for (int o = 0; o < 2; ++o) X[o] = mfma32(R.W[o][kk], Sb[kk], X[o]);
        // the decay of S ahead of the barrier, in the shadow of the X products (S is
        // not needed again before its update: its bf16 copy is already taken)
        const lds_float *scl = reinterpret_cast<const lds_float *>(eb + C::oS * 64);
        const float gl = scl[192];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
#pragma unroll
            for (int e = 0; e < 16; ++e) S[r][e] *= gl;
            asm volatile("" : "+v"(S[r]));   // keeps the scaling ahead of the barrier
        }
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                tX[((kh * 2 + (o ^ kh)) * 4 + j) * 64 + lane] =
                    __builtin_bit_cast(u32x4, f32x4{X[o][4 * j], X[o][4 * j + 1], X[o][4 * j + 2], X[o][4 * j + 3]});
        lds_barrier();                                        // B1
        if (ci + 2 < nch) load_w(R, ci + 2);
        // ---- U_new = X_0 + X_1; this wave publishes its own token tile of it, and takes
        // diag(d) U_new (rows in accumulator order) as the B operand of the update
        bf16x8 Ud[4];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const int m = o ^ kh;                             // the token tile
            f32x16 un, ud;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 xo = __builtin_bit_cast(f32x4, tX[(((kh ^ 1) * 2 + m) * 4 + j) * 64 + lane]);
                const f32x4 dj = *reinterpret_cast<const lds_f32x4 *>(scl + 32 * m + 8 * j + 4 * hh);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    un[4 * j + e] = X[o][4 * j + e] + xo[e];
                    ud[4 * j + e] = un[4 * j + e] * dj[e];
                }
            }
            Ud[2 * o] = pack32(ud, 0);
            Ud[2 * o + 1] = pack32(ud, 1);
            if (C::OUT && o == 0) {
                tU[(2 * kh) * 64 + lane] = __builtin_bit_cast(u32x4, pack32(un, 0));
                tU[(2 * kh + 1) * 64 + lane] = __builtin_bit_cast(u32x4, pack32(un, 1));
            }
        }
        // ---- own rows: S <- (2^(gam_n) S) + K^T diag(d) U_new
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int s = 0; s < 4; ++s) S[r] = mfma32(Kf[r][s], Ud[s], S[r]);
        lds_barrier();                                        // B2
    };
    for (int ci = 0; ci < nch; ci += 2) {
        chunk_step(ci, opA);
        if (ci + 1 < nch) chunk_step(ci + 1, opB);
    }

    if (!x.ptile) {
        if (p.sT) {
            float *dst = p.sT + unit * K * V;
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    dst[(int64_t)(row0 + 32 * r + 8 * (e >> 2) + 4 * hh + (e & 3)) * V + col] = S[r][e];
        }
    } else {
        // transition[i][j] = P[j][i]: P column pc is transition row pc
        const int pc = col - V;
        float *dst = p.trans + (unit * K + pc) * K + row0 + 4 * hh;
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4 *>(dst + 32 * r + 8 * j) =
                    f32x4{S[r][4 * j], S[r][4 * j + 1], S[r][4 * j + 2], S[r][4 * j + 3]};
    }
}

// The forward's workgroup (6 waves) takes 141 KiB of LDS at K = V = 128, one per CU (the
// two-tile one, 8 waves, 150 KiB).  The summary's (4 waves: no output waves) takes 63 KiB,
// two per CU.
template <int K, int V>
__global__ __launch_bounds__(384) void k_inter(Prob p, Ws w)
{
    static_assert(InterCfg<K, V, false>::THREADS == 384, "forward: 6 waves");
    inter_body<K, V, false>(p, w);
}

// The plain forward with two 32-column tiles per workgroup (8 waves, 150 KiB of LDS at
// K = V = 128): for batches that need more than one round of the one-tile workgroups.
template <int K, int V>
__global__ __launch_bounds__(512) void k_inter_wide(Prob p, Ws w)
{
    static_assert(InterCfg<K, V, false, 2>::THREADS == 512, "forward, two tiles: 8 waves");
    inter_body<K, V, false, false, false, false, 2>(p, w);
}

// The Gated Delta Product's forward: q rows and o rows mapped from update rows to
// tokens (a kernel of its own, so that the plain forward carries none of it).
template <int K, int V>
__global__ __launch_bounds__(384) void k_inter_gdp(Prob p, Ws w)
{
    inter_body<K, V, false, false, true>(p, w);
}

// The forward with the state series (a kernel of its own, so that the plain
// forward's chunk loop carries none of its stores).
template <int K, int V>
__global__ __launch_bounds__(384) void k_inter_ck(Prob p, Ws w)
{
    inter_body<K, V, false, true>(p, w);
}

// The same with two 32-column tiles per workgroup (8 waves), on the plain forward's terms.
template <int K, int V>
__global__ __launch_bounds__(512) void k_inter_ck_wide(Prob p, Ws w)
{
    static_assert(InterCfg<K, V, false, 2>::THREADS == 512, "forward, two tiles: 8 waves");
    inter_body<K, V, false, true, false, false, 2>(p, w);
}

// The backward's run of the forward: the fp32 state at every chunk start, no outputs, so no
// output waves and no q or P^T buffers (4 waves, 63 KiB of LDS at K = V = 128: two per CU).
template <int K, int V>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_inter_states(Prob p, Ws w)
{
    static_assert(InterCfg<K, V, false, 1, true>::THREADS == 256, "states only: 4 waves");
    inter_body<K, V, false, true, false, true>(p, w);
}

// The states only with two 32-column tiles per workgroup (6 waves, 82 KiB, one per CU): for
// batches that need more than one round of the CUs' one-tile workgroups.
template <int K, int V>
__global__ __launch_bounds__(384) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_inter_states_wide(Prob p, Ws w)
{
    static_assert(InterCfg<K, V, false, 2, true>::THREADS == 384, "states only, two tiles: 6 waves");
    inter_body<K, V, false, true, false, true, 2>(p, w);
}

template <int K, int V>
__global__ __launch_bounds__(256) void k_inter_sum(Prob p, Ws w)
{
    static_assert(InterCfg<K, V, true>::THREADS == 256, "summary: 4 waves");
    inter_body<K, V, true>(p, w);
}

// The summary with two 32-column tiles per workgroup (6 waves: four state waves, key half x
// tile, and the two loaders, the raw k rows shared; 82 KiB of LDS at K = V = 128, one
// workgroup per CU): for batches that need more than one round of the one-tile workgroups.
template <int K, int V>
__global__ __launch_bounds__(384) void k_inter_sum_wide(Prob p, Ws w)
{
    static_assert(InterCfg<K, V, true, 2>::THREADS == 384, "summary, two tiles: 6 waves");
    static_assert((V / 32) % 2 == 0, "the S and P columns split into whole pairs of tiles");
    inter_body<K, V, true, false, false, false, 2>(p, w);
}

// The Gated Delta Product's summary: k rows addressed by token and update.
template <int K, int V>
__global__ __launch_bounds__(256) void k_inter_sum_gdp(Prob p, Ws w)
{
    inter_body<K, V, true, false, true>(p, w);
}

// int64 cu_seqlens to the int32 copy the other kernels read (the "Linear Attention"
// page lists int64 offsets beside int32); entries outside the int32 range become -1,
// which the scheduler's validation reports as malformed.
__global__ __launch_bounds__(256) void k_cu64(const int64_t *src, int32_t *dst, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        const int64_t v = src[i];
        dst[i] = (v < 0 || v > INT32_MAX) ? -1 : (int32_t)v;
    }
}

hipError_t convert_cu64(const int64_t *src, int32_t *dst, int n, hipStream_t stream)
{
    if (n > 0) hipLaunchKernelGGL(k_cu64, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, src, dst, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host-side launch sequence.

namespace {

template <int K, int V, bool SUMMARY>
hipError_t launch_all(const Prob &p, const Ws &w, hipStream_t s, const LaunchHook *hook)
{
    auto before = [&](int id) { if (hook) hook->before(id, s, hook->ctx); };
    auto after = [&](int id) { if (hook) hook->after(id, s, hook->ctx); };

    // at most 64 sequences: the intra-chunk pass maps its own chunks and writes the tables
    if (p.N > 64) {
        before(LA_KERNEL_SCHED);
        hipLaunchKernelGGL(k_sched, dim3(1), dim3(1024), 0, s, p, w);
        after(LA_KERNEL_SCHED);
    }
    if (p.max_chunks > 0) {
        // persistent: at most three resident workgroups per CU, each walking (chunk, head) items
        const int64_t items = (int64_t)p.max_chunks * p.HV;
        const int grid = (int)(items < p.intra_grid ? items : p.intra_grid);
        before(LA_KERNEL_INTRA);
        if (p.nh > 1)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_intra<K, V, !SUMMARY, true>), dim3(grid), dim3(256), 0, s, p, w);
        else if (p.stream_ops)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_intra<K, V, !SUMMARY, false, 0, true>), dim3(grid), dim3(256), 0, s, p, w);
        else
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_intra<K, V, !SUMMARY, false>), dim3(grid), dim3(256), 0, s, p, w);
        after(LA_KERNEL_INTRA);
    }
    const int64_t blocks = (int64_t)p.N * p.HV * InterCfg<K, V, SUMMARY>::NT;
    if (blocks > 0) {
        before(LA_KERNEL_INTER);
        const dim3 threads(InterCfg<K, V, SUMMARY>::THREADS);
        if (SUMMARY && p.nh > 1)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_sum_gdp<K, V>), dim3((unsigned)blocks), threads, 0, s, p, w);
        else if (SUMMARY && (V / 32) % 2 == 0 && blocks > 2 * (p.intra_grid / 3))
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_sum_wide<K, V>), dim3((unsigned)(blocks / 2)),
                               dim3(InterCfg<K, V, true, 2>::THREADS), 0, s, p, w);
        else if (SUMMARY)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_sum<K, V>), dim3((unsigned)blocks), threads, 0, s, p, w);
        else if (p.nh > 1)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_gdp<K, V>), dim3((unsigned)blocks), threads, 0, s, p, w);
        else if (p.ck_every > 0 && blocks > p.intra_grid / 3 && blocks <= 2 * (p.intra_grid / 3))
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_ck_wide<K, V>), dim3((unsigned)(blocks / 2)),
                               dim3(InterCfg<K, V, false, 2>::THREADS), 0, s, p, w);
        else if (p.ck_every > 0)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_ck<K, V>), dim3((unsigned)blocks), threads, 0, s, p, w);
        else if (blocks > p.intra_grid / 3 && blocks <= 2 * (p.intra_grid / 3))
            // one-tile workgroups (one fits a CU) for up to two rounds of the CUs: two tiles
            // per workgroup, one round, each chunk step about 1.6x as long (dense batch of 8 x
            // 4096 tokens, HV = 16: 202 -> 162 us).  With more rounds the longest sequence's
            // chain decides, and its steps are shorter with one tile (the ragged batch with a
            // 65,536-token sequence, H = 32: 2478 us with one tile, 2536 us with two).
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_wide<K, V>), dim3((unsigned)(blocks / 2)),
                               dim3(InterCfg<K, V, false, 2>::THREADS), 0, s, p, w);
        else
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter<K, V>), dim3((unsigned)blocks), threads, 0, s, p, w);
        after(LA_KERNEL_INTER);
    }
    return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// k_bwd_inter: the reverse chunk pass of the backward, and the span summary's mirror for the
// state gradient (the "Linear Attention" page, "Summaries": <op>_summary_bwd).  With
// L = sum_t <dO_t, o_t> + <dS_end, S_end>, the gradient dS of a chunk's end state gives
// that of its start state (the chunked form of the forward's formulas at the top, read
// backwards):
//     dU  = diag(d) K dS + P^T dO                      (d = 2^(gam_n - gam) r_k)
//     dS0 = 2^(gam_n) dS + Q^T diag(sq) dO + (-W)^T dU  (sq = scale r_q 2^gam)
// One workgroup of 4 waves per (sequence, value head, 32 value columns), over the chunks
// from last to first:
//   state waves kh = 0, 1 own the rows of key half kh of dS (accumulator tiles) and carry
//     the chain: Z_kh = K_kh dS_kh over both token tiles (their half of the reduction over
//     keys), swapped through LDS so that both hold dU; the P^T dO and Q^T diag(sq) dO
//     terms, which do not depend on dS, are formed before the swap.  They read every
//     operand from LDS and issue no loads, so no wait of theirs covers a load in flight.
//   loader waves (2, 3) put chunk c - 1's raw k, q and dO rows, scalars, and -W^T and P^T
//     fragments (written by the intra pass in this pass's operand order) into LDS at the
//     start of chunk c (two buffers) and wait for them before the chunk's second barrier.
// FULL (the full backward) also stores each chunk's end-state gradient and dU for the
// backward's intra pass.
// TP = 2: two 32-column tiles per workgroup (four state waves, key half x tile, and the two
// loaders; the k, q, -W^T and P^T operands shared), for batches that would need more than
// one round of the one-tile workgroups (158 KiB of LDS at K = V = 128).

template <int K, int V, bool FULL, int TP = 1>
__global__ __launch_bounds__(64 * (2 * TP + 2)) __attribute__((amdgpu_waves_per_eu(TP, TP))) void k_bwd_inter(
    Prob p, Ws w, const __bf16 *d_out, const float *d_end, float *d_start)
{
    constexpr int KH = K / 2, NR = KH / 32, NKS = KH / 16, PPR = K / 8;
    constexpr int NT = V / 32 / TP;              // workgroups per (sequence, head)
    constexpr int FK = K / 8;                    // fragments of a 64-row k or q tile
    constexpr int NKL = FK / 2;                  // k (or q) tile loads per loader wave
    constexpr int FWT = (K / 32) * 4;            // -W^T fragments per chunk
    constexpr int oK = 0, oQ = FK, oD = 2 * FK, oS = oD + 4 * TP, oWT = oS + 1, oPT = oWT + FWT, NF = oPT + 6;
    constexpr int SW = 2 * TP;                   // state waves; the loaders are waves SW, SW + 1
    __shared__ u32x4 sB0[NF * 64], sB1[NF * 64];
    __shared__ u32x4 sZ[TP * 2 * 2 * 4 * 64];   // Z partials: [tile][kh][token tile][j][lane]
    lds_u32x4 *const b0 = (lds_u32x4 *)sB0, *const b1 = (lds_u32x4 *)sB1;
    auto buf = [&](int c) { return (c & 1) ? b1 : b0; };
    lds_u32x4 *const xZ = (lds_u32x4 *)sZ;

    if (w.hdr[0] != LA_DEVICE_OK) return;        // malformed cu_seqlens: write nothing
    const UnitOfBlock ub = unit_of_block(p, w, blockIdx.x, NT);   // as the forward
    const int n = ub.n, h = ub.h, tile = ub.tile;
    const int hk = h / (p.HV / p.HK);
    const int4 si = w.seq_info[n];
    const int seq_start = si.x, seq_len = si.y, cid0 = si.z;
    const int nch = (seq_len + kChunk - 1) / kChunk;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 31, hh = lane >> 5;

    if (wave >= SW) {
        // ------------------------------------------------------------ loader waves
        const int lh = wave - SW;
        uint32_t koff[NKL], qoff[NKL], doff[2];
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int sI = (2 * i + lh) * 64 + lane;
            const int row = sI / PPR, pc = (sI % PPR) ^ swz_mask<PPR>(row);
            koff[i] = (uint32_t)row * 2u * (uint32_t)p.kst + 16u * (uint32_t)pc;
            qoff[i] = (uint32_t)row * 2u * (uint32_t)p.qst + 16u * (uint32_t)pc;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int sI = (2 * i + lh) * 64 + lane;
            const int row = sI / 4, pc = (sI % 4) ^ swz_mask<4>(row);
            doff[i] = (uint32_t)row * 2u * (uint32_t)p.ost + 16u * (uint32_t)pc;
        }
        const uint32_t lo16 = (uint32_t)lane * 16u;
        // chunk ci's k, q and dO rows, scalars, -W^T and P^T fragments into `eb`
        auto issue = [&](lds_u32x4 *eb, int ci) {
            const int start = seq_start + kChunk * ci, len = min(kChunk, seq_len - kChunk * ci);
            const int64_t chh = (int64_t)(cid0 + ci) * p.HV + h;
            const i32x4 rK = make_rsrc(p.k + (int64_t)start * p.kst + (int64_t)hk * p.ksh, (uint32_t)len * 2u * (uint32_t)p.kst);
#pragma unroll
            for (int i = 0; i < NKL; ++i) b2l(rK, eb, oK + 2 * i + lh, koff[i], 0);
            const i32x4 rQ = make_rsrc(p.q + (int64_t)start * p.qst + (int64_t)hk * p.qsh, (uint32_t)len * 2u * (uint32_t)p.qst);
#pragma unroll
            for (int i = 0; i < NKL; ++i) b2l(rQ, eb, oQ + 2 * i + lh, qoff[i], 0);
#pragma unroll
            for (int tp = 0; tp < TP; ++tp) {
                const i32x4 rD = make_rsrc(d_out + (int64_t)start * p.ost + (int64_t)h * p.osh + 32 * (TP * tile + tp),
                                           (uint32_t)len * 2u * (uint32_t)p.ost);
#pragma unroll
                for (int i = 0; i < 2; ++i) b2l(rD, eb, oD + 4 * tp + 2 * i + lh, doff[i], 0);
            }
            const i32x4 rW = make_rsrc(reinterpret_cast<const char *>(w.WTF) + chh * FWT * kFrag, FWT * kFrag);
#pragma unroll
            for (int i = 0; i < FWT / 2; ++i) {
                const int f = lh * (FWT / 2) + i;
                b2l(rW, eb, oWT + f, lo16, f * kFrag);
            }
            const i32x4 rP = make_rsrc(reinterpret_cast<const char *>(w.PTF) + chh * 6 * kFrag, 6 * kFrag);
#pragma unroll
            for (int i = 0; i < 3; ++i) b2l(rP, eb, oPT + 3 * lh + i, lo16, (3 * lh + i) * kFrag);
            if (lh == 0) b2l(make_rsrc(w.SC + chh * kScalars, kScalars * 4), eb, oS, lo16, 0);
        };
        // Chunk ci's operands land in buffer ci % 2.  At the start of chunk ci (after B2 of chunk
        // ci + 1, whose buffer is then dead) the loaders issue chunk ci - 1's; before B2 of
        // chunk ci they wait for them.
        if (nch > 0) issue(buf(nch - 1), nch - 1);
        vm_wait<0>();
        lds_barrier();
        for (int ci = nch - 1; ci >= 0; --ci) {
            if (ci >= 1) issue(buf(ci - 1), ci - 1);
            lds_barrier();                                    // B1
            vm_wait<0>();                                     // all of chunk ci - 1
            lds_barrier();                                    // B2
        }
        return;
    }

    // ---------------------------------------------------------------- state waves
    __builtin_amdgcn_s_setprio(3);
    const int kh = wave & 1, tp = wave >> 1;
    const int row0 = kh * KH;                            // first key row of this wave
    const int col = 32 * (TP * tile + tp) + c;           // this lane's value column
    lds_u32x4 *const tZ = xZ + tp * (2 * 2 * 4 * 64);     // this tile's Z partials
    const int64_t unit = (int64_t)n * p.HV + h;
    f32x16 D[NR];                                        // dS rows row0 .. row0 + KH - 1
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            D[r][e] = d_end ? d_end[(unit * K + row0 + 32 * r + 8 * (e >> 2) + 4 * hh + (e & 3)) * V + col] : 0.f;
    // chunk cj's end-state gradient (dS as it enters chunk cj's step), for the backward's intra
    // pass in the row-quad layout.  Stored at the end of chunk cj + 1's step (the last chunk's
    // before the loop), when the loaders' operand loads have landed: stored at the start of the
    // step, beside the loaders' next issue, the stores delayed those loads (dense batch 440 ->
    // 398 us).
    auto store_dsn = [&](int cj) {
        if (FULL) {
            float *dst = w.DSN + ((int64_t)(cid0 + cj) * p.HV + h) * K * V;
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<f32x4 *>(dst + quad_off(row0 + 32 * r + 8 * j + 4 * hh, col, V)) =
                        f32x4{D[r][4 * j], D[r][4 * j + 1], D[r][4 * j + 2], D[r][4 * j + 3]};
        }
    };
    if (nch > 0) store_dsn(nch - 1);
    lds_barrier();
    for (int ci = nch - 1; ci >= 0; --ci) {
        const lds_u32x4 *eb = buf(ci);
        const lds_u32x2 *ew = reinterpret_cast<const lds_u32x2 *>(eb);
        const lds_float *scl = reinterpret_cast<const lds_float *>(eb + oS * 64);
        const int64_t chh = (int64_t)(cid0 + ci) * p.HV + h;
        // dS as bf16 B operands (keys in accumulator order)
        bf16x8 Sb[NKS];
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) Sb[kk] = pack32(D[kk >> 1], kk & 1);
        // Z[o] = K (token tile m = o ^ kh, keys of this half) dS_kh; A operands are k rows with the
        // keys in accumulator order (two 8-byte reads of the swizzled tile)
        f32x16 Z[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            Z[o] = f32x16{};
            const int rowt = 32 * (o ^ kh) + c;
#pragma unroll
            for (int kk = 0; kk < NKS; ++kk) {
                const int ck = row0 + 16 * kk + 4 * hh;
                const u32x2 a0 = ew[oK * 128 + (swz<PPR>(rowt, ck) >> 3)];
                const u32x2 a1 = ew[oK * 128 + (swz<PPR>(rowt, ck + 8) >> 3)];
                Z[o] = mfma32(__builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]}), Sb[kk], Z[o]);
            }
        }
        // dO as B operands (tokens in accumulator order), token steps 0..3
        bf16x8 Do[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) Do[st] = lds_tr32s<4, true>(eb + (oD + 4 * tp) * 64, 16 * st, 0, lane);
        // G2 = P^T dO for both token tiles (P causal: s tile m needs t tiles m .. 1)
        f32x16 Gz[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const int m = o ^ kh;
            Gz[o] = f32x16{};
#pragma unroll
            for (int pt = 0; pt < 2; ++pt)
                if (pt >= m) {
#pragma unroll
                    for (int js = 0; js < 2; ++js)
                        Gz[o] = mfma32(__builtin_bit_cast(bf16x8, eb[(oPT + 2 * (m + pt) + js) * 64 + lane]), Do[2 * pt + js],
                                       Gz[o]);
                }
        }
        // the decay of dS, then Q^T diag(sq) dO of this key half
        const float gl = scl[192];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int e = 0; e < 16; ++e) D[r][e] *= gl;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const f32x4 s0 = *reinterpret_cast<const lds_f32x4 *>(scl + 64 + 16 * st + 4 * hh);
            const f32x4 s1 = *reinterpret_cast<const lds_f32x4 *>(scl + 64 + 16 * st + 8 + 4 * hh);
            bf16x8 Ds;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Ds[i] = f2bf(bf2f(Do[st][i]) * s0[i]);
                Ds[4 + i] = f2bf(bf2f(Do[st][4 + i]) * s1[i]);
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) D[r] = mfma32(lds_tr32s<PPR, true>(eb + oQ * 64, 16 * st, row0 + 32 * r, lane), Ds, D[r]);
        }
        // swap the Z partials
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                tZ[((kh * 2 + (o ^ kh)) * 4 + j) * 64 + lane] =
                    __builtin_bit_cast(u32x4, f32x4{Z[o][4 * j], Z[o][4 * j + 1], Z[o][4 * j + 2], Z[o][4 * j + 3]});
        lds_barrier();                                        // B1
        // dU = diag(d) (Z_0 + Z_1) + P^T dO for both token tiles (own tile first: only addresses
        // depend on kh, never a register index); D += (-W)^T dU
        bf16x8 Ub[2][2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const int m = o ^ kh;
            f32x16 du;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 zo = __builtin_bit_cast(f32x4, tZ[(((kh ^ 1) * 2 + m) * 4 + j) * 64 + lane]);
                const f32x4 dj = *reinterpret_cast<const lds_f32x4 *>(scl + 32 * m + 8 * j + 4 * hh);
#pragma unroll
                for (int e = 0; e < 4; ++e) du[4 * j + e] = (Z[o][4 * j + e] + zo[e]) * dj[e] + Gz[o][4 * j + e];
            }
            Ub[o][0] = pack32(du, 0);
            Ub[o][1] = pack32(du, 1);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int o = 0; o < 2; ++o)
#pragma unroll
                for (int js = 0; js < 2; ++js)
                    D[r] = mfma32(__builtin_bit_cast(bf16x8, eb[(oWT + (kh * NR + r) * 4 + 2 * (o ^ kh) + js) * 64 + lane]),
                                  Ub[o][js], D[r]);
        if (FULL) {
            // dU of this wave's token tile in bf16 (the operand precision the backward's intra
            // pass reads it in), from its packed operands, at the end of the step like dS
            __bf16 *dst = w.DU + (chh * 64 + 32 * kh) * V + col;
#pragma unroll
            for (int e = 0; e < 16; ++e) dst[(int64_t)(8 * (e >> 2) + 4 * hh + (e & 3)) * V] = Ub[0][e >> 3][e & 7];
        }
        if (ci >= 1) store_dsn(ci - 1);
        lds_barrier();                                        // B2
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            d_start[(unit * K + row0 + 32 * r + 8 * (e >> 2) + 4 * hh + (e & 3)) * V + col] = D[r][e];
}

// ---------------------------------------------------------------------------
// k_bwd_intra: the backward's intra pass, one workgroup of 4 waves per (chunk, value head).
// Given the chunk's start state S0 (the recomputed forward's fp32 series), the gradient dS
// of its end state and dU (both from the reverse pass), it differentiates everything the
// forward formed inside the chunk (the formulas at the top of this file; k^ = r_k k and
// q^ = scale r_q q, f = beta 2^gam, M[t][s] = 2^(gam_t - gam_s) for s <= t):
//   U   = U~ + (-W) S0                       dP  = dO U^T
//   dq^ = diag(2^gam) dO S0^T + (M o dP) k^  dk^ = (M o dP)^T q^ + diag(2^(gam_n-gam)) U dS^T
//   dW  = -dU S0^T                           dT  = dW (diag(f) k^)^T + dU (diag(beta) V)^T
//   dk^ += diag(f) T^T dW                    dv  = diag(beta) T^T dU
//   dA  = -T^T (dT T^T), strictly lower      dk^ += (dGm + dGm^T) k^,  dGm = dA o beta_t E
// with E[t][s] = 2^(gam_t - gam_s) (s < t), and per token the gradients of beta and of the
// chunk-local cumulative gate (every place gam enters: A, P, W, the output's 2^gam, the
// state update's 2^(gam_n - gam) and 2^gam_n), summed back to g in reverse token order.
// The q^ and k^ gradients go out per value head (fp32) and k_bwd_qk sums each head group and
// applies the row norms; with one value head per q/k head, or (GL) a whole head group per
// workgroup, this kernel applies them itself.  All products are bf16 MFMA with fp32 accumulation; each wave owns
// token tile (wave & 1) and the column tiles (wave >> 1) + 2 i of every 64-row result.  At
// K = V = 128 the workgroup is 8 waves (two per SIMD, the only workgroup on its CU): waves w
// and w + 4 split the K- and V-wide products by column tile and take the 64 x 64 ones
// (dT and Y; dP, P, the Gram tile and dA) by product, so that a phase's chain of dependent
// LDS reads and products is about half as long per wave.
// Stage A holds S0 and dS in LDS (bf16); stage B reuses that space for q, v, T and the
// masked dP tiles; stage C for dT T^T and the dA tiles.

template <int PPR>
__device__ __forceinline__ int swz_e(int row, int col)
{
    return swz<PPR>(row, col & ~3) + 2 * (col & 3);
}

// Row sums of an accumulator tile: register e of every lane summed over the 32 lanes that
// share lane >> 5 (the 32 columns of the tile's row 8 (e >> 2) + 4 hh + (e & 3)), for all 16
// registers at once.  Each step exchanges half of the remaining values with a partner lane
// that differs in the next lane bit (masks 16, 15, 7, 2, 1: independent, so the partial sums
// cover all 32 lanes) and keeps the half that bit selects; lane c ends with the sum of
// register c >> 1 (the same bits in lanes c and c ^ 1).  16 exchanges instead of 80.
__device__ __forceinline__ float rowsum32(const float (&v)[16], int lane)
{
    const int c = lane & 31;
    const bool b4 = c & 16, b3 = c & 8, b2 = c & 4, b1 = c & 2;
    float a[8], b[4], d[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (b4 ? v[i + 8] : v[i]) + xch16(b4 ? v[i] : v[i + 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (b3 ? a[i + 4] : a[i]) + xch15(b3 ? a[i] : a[i + 4]);
#pragma unroll
    for (int i = 0; i < 2; ++i) d[i] = (b2 ? b[i + 2] : b[i]) + xch7(b2 ? b[i] : b[i + 2]);
    const float e = (b1 ? d[1] : d[0]) + xch2(b1 ? d[0] : d[1]);
    return e + xch1(e);
}

// A 32 x 32 accumulator tile (rows r0 + 8 j + 4 hh + i in register 4 j + i, column c0 + lane % 32)
// into a swizzled bf16 tile of PPR 16-byte pieces per row.
template <int PPR>
__device__ __forceinline__ void store_tile_bf16(lds_char *tile, const f32x16 &x, int r0, int c0, int lane)
{
    const int c = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        *reinterpret_cast<lds_bf16 *>(tile + swz_e<PPR>(r0 + 8 * (e >> 2) + 4 * hh + (e & 3), c0 + c)) = f2bf(x[e]);
}

template <int PPR>
__device__ __forceinline__ float lds_elem(const lds_char *tile, int row, int col)
{
    return bf2f(*reinterpret_cast<const lds_bf16 *>(tile + swz_e<PPR>(row, col)));
}

// The 16 elements of a swizzled bf16 tile that an accumulator lane (c, hh) holds of a 32 x 32
// block (rows r0 + 8 j + 4 hh + i in register 4 j + i, column c0 + c; r0 and c0 multiples of
// 32): two transposed reads in accumulator order instead of 16 two-byte reads.
template <int PPR>
__device__ __forceinline__ void acc_elems(const lds_char *tile, int r0, int c0, int lane, float (&x)[16])
{
    const bf16x8 a = lds_tr32s<PPR, true>(reinterpret_cast<const lds_u32x4 *>(tile), r0, c0, lane);
    const bf16x8 b = lds_tr32s<PPR, true>(reinterpret_cast<const lds_u32x4 *>(tile), r0 + 16, c0, lane);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = bf2f(a[e]);
        x[8 + e] = bf2f(b[e]);
    }
}

// The backward intra pass's fp32 operands S0 (row-major, or in the row-quad layout for
// S0_QUAD) and dS (row-quad layout) into swizzled bf16 tiles, by the NT threads of the block
// in 4 x 4 blocks (four 16-byte loads of each matrix per block), with every load issued
// before the first is used (one memory latency instead of one per batch).  Returns the
// thread's share of sum(S0 * dS), summed in the same order for either S0 layout.
template <int K, int V, bool S0_QUAD, int NT>
__device__ __forceinline__ float load_stage_a(lds_char *dS0, const float *S0, lds_char *dDS, const float *DS, int tid)
{
    constexpr int PPR = V / 8, NB = K * V / 16 / NT;
    static_assert(NB * NT * 16 == K * V, "whole 4 x 4 blocks per thread");
    float4 a[NB][4], b[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int blk = tid + NT * j, rq = blk / (V / 4), c4 = 4 * (blk % (V / 4));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // S0_QUAD: column c4 + u, rows 4 rq .. 4 rq + 3; else row 4 rq + u, columns c4 .. c4 + 3
            a[j][u] = *reinterpret_cast<const float4 *>(S0 + (S0_QUAD ? ((int64_t)rq * V + c4 + u) * 4
                                                                      : (int64_t)(4 * rq + u) * V + c4));
            b[j][u] = *reinterpret_cast<const float4 *>(DS + ((int64_t)rq * V + c4 + u) * 4);
        }
    }
    auto el = [](const float4 &x, int i) { return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w; };
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int blk = tid + NT * j, rq = blk / (V / 4), c4 = 4 * (blk % (V / 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s[4], d[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                s[u] = S0_QUAD ? el(a[j][u], i) : el(a[j][i], u);
                d[u] = el(b[j][u], i);
                dot += s[u] * d[u];
            }
            const int row = 4 * rq + i;
            *reinterpret_cast<lds_bf16x4 *>(dS0 + swz<PPR>(row, c4)) = bf16x4{f2bf(s[0]), f2bf(s[1]), f2bf(s[2]), f2bf(s[3])};
            *reinterpret_cast<lds_bf16x4 *>(dDS + swz<PPR>(row, c4)) = bf16x4{f2bf(d[0]), f2bf(d[1]), f2bf(d[2]), f2bf(d[3])};
        }
    }
    return dot;
}

template <int K, int V, int NW, bool GL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void k_bwd_intra(
    Prob p, Ws w, const __bf16 *d_out, float *dv_out, float *dg_out, float *db_out, float *dq_out, float *dk_out)
{
    constexpr int PK = K / 8, PV = V / 8, NKT = K / 32, NVT = V / 32, KS = K / 16, VS = V / 16;
    // NW = 8: two waves per (token tile, column tile) pair, which split the K- and V-wide
    // products by column tile (IK, IV per wave) and share the 64 x 64 ones by product
    static_assert(NW == 4 || (NW == 8 && NKT % 4 == 0 && NVT % 4 == 0), "8 waves need K and V in multiples of 128");
    static_assert(!GL || NW == 8, "the head-group loop runs on the 8-wave workgroup");
    constexpr int NQ = NW / 4, IK = NKT / (2 * NQ), IV = NVT / (2 * NQ);
    constexpr int NKS = K / 32;                             // steps of 16 keys per key half (-W fragments)
    constexpr int szK = 64 * K * 2, szV = 64 * V * 2, sz64 = 64 * 64 * 2, szS = K * V * 2;
    constexpr int R1B = 2 * szS > szK + szV + 4 * sz64 ? 2 * szS : szK + szV + 4 * sz64;
    constexpr int oK = 0, oDO = oK + szK, oR1 = oDO + szV, oDU = oR1 + R1B, oU = oDU + szV, oDW = oU + szV;
    constexpr int oEnd = oDW + szK;
    constexpr int oS0 = oR1, oDS = oR1 + szS;                            // stage A
    constexpr int oQ = oR1, oVv = oQ + szK, oT = oVv + szV, oR = oT + sz64, oR2 = oR + sz64, oDT = oR2 + sz64;
    constexpr int oY = oQ, oZ = oVv, oZ3 = oR;                           // stage C
    enum { XV, DF, DAEG, AAR, AAC, PPR_, PPC, QX, KX, QD, KD, NPART };
    __shared__ __attribute__((aligned(16))) char smem[oEnd];
    __shared__ __attribute__((aligned(16))) float ssc[6 * 64];   // gam2, r_k, r_q, beta, 2^gam, 2^(gam_n - gam)
    __shared__ float part[NPART][2 * NQ][64];   // per-token partial sums: [column tile half + 2 qw] or [tile]
    __shared__ float sdot[NW];
    __shared__ float pf_sink[NW == 8 ? NW * 64 : 1];   // landing slots of the next item's cache-line touches
    lds_char *const L = (lds_char *)smem;
    const lds_u32x4 *const tK = (const lds_u32x4 *)(L + oK);
    const lds_u32x4 *const tDO = (const lds_u32x4 *)(L + oDO);
    const lds_u32x4 *const tDU = (const lds_u32x4 *)(L + oDU);
    const lds_u32x4 *const tU = (const lds_u32x4 *)(L + oU);
    const lds_u32x4 *const tDW = (const lds_u32x4 *)(L + oDW);
    const lds_u32x4 *const tS0 = (const lds_u32x4 *)(L + oS0);
    const lds_u32x4 *const tDS = (const lds_u32x4 *)(L + oDS);
    const lds_u32x4 *const tQ = (const lds_u32x4 *)(L + oQ);
    const lds_u32x4 *const tV = (const lds_u32x4 *)(L + oVv);
    const lds_u32x4 *const tT = (const lds_u32x4 *)(L + oT);
    const lds_u32x4 *const tR = (const lds_u32x4 *)(L + oR);
    const lds_u32x4 *const tR2 = (const lds_u32x4 *)(L + oR2);
    const lds_u32x4 *const tDT = (const lds_u32x4 *)(L + oDT);
    const lds_u32x4 *const tY = (const lds_u32x4 *)(L + oY);
    const lds_u32x4 *const tZ = (const lds_u32x4 *)(L + oZ);
    const lds_u32x4 *const tZ3 = (const lds_u32x4 *)(L + oZ3);
    lds_float *const s_gam = (lds_float *)ssc, *const s_rk = s_gam + 64, *const s_rq = s_gam + 128;
    lds_float *const s_b = s_gam + 192, *const s_eg = s_gam + 256, *const s_dd = s_gam + 320;

    if (w.hdr[0] != LA_DEVICE_OK) return;
    const int lane0 = threadIdx.x & 63;
    // the item: chunk ci of the chunk table and value head h0; GL: q/k head hk and its G value
    // heads h0 .. h0 + G - 1, one after another, with dq^ and dk^ summed over them in registers
    const int G = p.HV / p.HK, NH = GL ? G : 1;
    const int ci = GL ? (int)blockIdx.x / p.HK : (int)blockIdx.x / p.HV;
    const int hk = GL ? (int)blockIdx.x % p.HK : ((int)blockIdx.x % p.HV) / G;
    const int h0 = GL ? hk * G : (int)blockIdx.x % p.HV;
    int start, len, total;
    if (p.N <= 64) {
        const SmallMap sm = small_map(p, w, false);
        total = sm.total;
        if (ci >= sm.total) return;
        const uint64_t owns = __ballot(lane0 < p.N && sm.first <= ci);
        const int sq_ = 63 - __builtin_clzll(owns);
        start = __builtin_amdgcn_readfirstlane(__shfl(sm.start, sq_, 64) + kChunk * (ci - __shfl(sm.first, sq_, 64)));
        len = __builtin_amdgcn_readfirstlane(min(kChunk, __shfl(sm.end, sq_, 64) - start));
    } else {
        total = w.hdr[1];
        if (ci >= total) return;
        const int4 ch = w.chunks[ci];
        start = __builtin_amdgcn_readfirstlane(ch.y);
        len = __builtin_amdgcn_readfirstlane(ch.z);
    }
    // With several rounds of items (one workgroup per CU), the first round starts in 8 phases
    // about an eighth of an item apart (blocks 8 apart share an XCD, so each XCD gets every
    // phase): the CUs then run their items back to back out of step, instead of all issuing
    // their ~200 KiB of stage-A loads at the same moment of every round.  With 4 waves at
    // K = V = 128 (about 34 us per item) a phase step of 127 x 64 clocks took the varlen
    // backward from 168 to 152 us and the dense batch from 1081 to 1019 us (8 phases of 64 x 64
    // clocks gained less, 16 or 32 phases of 127 x 64 clocks lost part of it again); the
    // 8-wave items (about 25 us per value head) take 96 x 64 per head (64: 132 -> 124 us
    // varlen; 127 or 160: slower).  Single-round launches start at once.
    if ((int)gridDim.x > 2 * (p.intra_grid / 3) && (int)blockIdx.x < p.intra_grid / 3) {
        constexpr int STEP = NW == 8 ? 96 : (K * V >= 8192 ? 64 : 32);
        const int ph = ((int)blockIdx.x >> 3) & 7;
        for (int i = 0; i < ph * NH; ++i) __builtin_amdgcn_s_sleep(STEP);
    }
    const bool fuse_qk = dq_out != nullptr;
    f32x16 dQ[IK], dK[IK];   // dq^ and dk^ (GL: summed over the heads done so far)
    // GL: this lane's row dot of q with dq^ as the previous heads left it (the output's state
    // term of this head's dgam is the row dot of q with what this head's A2 adds to it)
    float qprev = 0.f;
    for (int j = 0; j < NH; ++j) {
    // GL: the thread and wave indices pass through an empty asm per head, so that the compiler
    // forms the many lane-dependent LDS addresses of a head inside the loop instead of hoisting
    // them all out of it, where they would stay live across the whole loop (and spill)
    int tid_ = threadIdx.x, wave_ = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (GL) asm volatile("" : "+v"(tid_), "+s"(wave_));
    const int tid = tid_, lane = tid & 63, c = lane & 31, hh = lane >> 5, wave = wave_;
    const int tm = wave & 1, half = (wave >> 1) & 1, qw = wave >> 2, pw = half + 2 * qw;
    // 64 x 64 products: dT (A5, B3) and Y (C1) on the waves with qw = 0, dP (B1, B2), the
    // Gram tile and dA (C2) on those with qw = 1 (all on the one set of 4 waves for NW = 4)
    const bool wT = NQ == 1 || qw == 0, wP = NQ == 1 || qw == 1;
    // the wave's i-th column tile of a K- or V-wide result
    auto ctile = [&](int i) { return half + 2 * (NQ * i + qw); };
    __bf16 xq[IK][16];   // the q elements of this lane's dq^ entries, for the chain rule below
    const int h = h0 + j;
    const int64_t chh = (int64_t)ci * p.HV + h;

    // ---- stage A loads: k (once per item), dO and dU rows (buffer loads into LDS), the
    // scalars, S0 and dS
    if (j == 0)
        intra_load_tile<K>((lds_u32x4 *)(L + oK), p.k + (int64_t)start * p.kst + (int64_t)hk * p.ksh,
                           2u * (uint32_t)p.kst, len, wave, lane, NW);
    intra_load_tile<V>((lds_u32x4 *)(L + oDO), d_out + (int64_t)start * p.ost + (int64_t)h * p.osh,
                       2u * (uint32_t)p.ost, len, wave, lane, NW);
    intra_load_tile<V>((lds_u32x4 *)(L + oDU), w.DU + chh * 64 * V, 2u * (uint32_t)V, 64, wave, lane, NW);
    // A1's register operands (-W fragments, the U~ tiles and their scales), issued with the rest
    bf16x8 Wf[KS];
    uint2 uh[IV][4];
    int ush[IV];
#pragma unroll
    for (int kg = 0; kg < KS; ++kg)
        Wf[kg] = __builtin_bit_cast(bf16x8, w.WF[(chh * (K / 8) + ((kg / NKS) * 2 + tm) * NKS + kg % NKS) * 64 + lane]);
#pragma unroll
    for (int i = 0; i < IV; ++i) {
        const int vt = ctile(i);
        ush[i] = __float_as_int(w.SC[chh * kScalars + 128 + 2 * vt + tm]);
#pragma unroll
        for (int j = 0; j < 4; ++j) uh[i][j] = w.UH[(((chh * (V / 32) + vt) * 2 + tm) * 4 + j) * 64 + lane];
    }
    if (tid < 64) {
        const float *sb = w.SB + chh * kScalars;
        const float gam = sb[tid], gn = sb[len - 1];
        s_gam[tid] = gam;
        s_rk[tid] = sb[64 + tid];
        s_rq[tid] = sb[128 + tid];
        s_b[tid] = sb[192 + tid];
        s_eg[tid] = exp2_hw(gam);
        s_dd[tid] = exp2_hw(tid < len ? gn - gam : kNegInf);
    }
    float dot = p.ck_quad ? load_stage_a<K, V, true, 64 * NW>(L + oS0, w.CK + chh * K * V, L + oDS, w.DSN + chh * K * V, tid)
                          : load_stage_a<K, V, false, 64 * NW>(L + oS0, w.CK + chh * K * V, L + oDS, w.DSN + chh * K * V, tid);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (lane == 0) sdot[wave] = dot;
    vm_wait<0>();
    lds_barrier();

    // ---- A1: U = U~ + (-W) S0 for tiles (tm, value tile half + 2 i); U~ enters the accumulator
    {
#pragma unroll
        for (int i = 0; i < IV; ++i) {
            const int vt = ctile(i);
            f32x16 acc;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 u4 = f16_unpack4(__builtin_bit_cast(u32x2, uh[i][j]), ush[i]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[4 * j + e] = u4[e];
            }
#pragma unroll
            for (int kg = 0; kg < KS; ++kg) acc = mfma32(Wf[kg], lds_tr32s<PV, true>(tS0, 16 * kg, 32 * vt, lane), acc);
            store_tile_bf16<PV>(L + oU, acc, 32 * tm, 32 * vt, lane);
        }
    }
    // ---- A2, A4: dO S0^T (the output's state term of dq^, rows scaled by 2^gam) and dW = -dU S0^T
#pragma unroll
    for (int i = 0; i < IK; ++i) {
        const int kt = ctile(i);
        f32x16 a = {}, b = {};
#pragma unroll
        for (int s = 0; s < VS; ++s) {
            const bf16x8 sv = lds_row8<PV>(tS0, 32 * kt + c, 16 * s + 8 * hh);
            a = mfma32(lds_row8<PV>(tDO, 32 * tm + c, 16 * s + 8 * hh), sv, a);
            b = mfma32(lds_row8<PV>(tDU, 32 * tm + c, 16 * s + 8 * hh), sv, b);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            a[e] *= s_eg[32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3)];
            b[e] = -b[e];
        }
        dQ[i] = GL && j > 0 ? dQ[i] + a : a;
        store_tile_bf16<PK>(L + oDW, b, 32 * tm, 32 * kt, lane);
    }
    lds_barrier();                                            // U and dW published
    // ---- A3: diag(2^(gam_n - gam)) U dS^T (the state update's term of dk^), and F = its row dot with k^
    {
        float prod[16] = {};
#pragma unroll
        for (int i = 0; i < IK; ++i) {
            const int kt = ctile(i);
            f32x16 a = {};
#pragma unroll
            for (int s = 0; s < VS; ++s)
                a = mfma32(lds_row8<PV>(tU, 32 * tm + c, 16 * s + 8 * hh), lds_row8<PV>(tDS, 32 * kt + c, 16 * s + 8 * hh), a);
            float xk[16];
            acc_elems<PK>(L + oK, 32 * tm, 32 * kt, lane, xk);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
                a[e] *= s_dd[row];
                prod[e] += a[e] * xk[e];
            }
            dK[i] = GL && j > 0 ? dK[i] + a : a;
        }
        {
            const float r = rowsum32(prod, lane);
            const int e = c >> 1, row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
            if ((c & 1) == 0) part[KX][pw][row] = r * s_rk[row];
        }
    }
    // ---- A5, B1: dT's first term dW (diag(f r_k) K)^T and dP = dO U^T, tile (tm, half)
    f32x16 dT = {}, dP = {};
    if (wT) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            dT = mfma32(lds_row8<PK>(tDW, 32 * tm + c, 16 * s + 8 * hh), lds_row8<PK>(tK, 32 * half + c, 16 * s + 8 * hh), dT);
        const int sc_ = 32 * half + c;
        const float fr = s_b[sc_] * s_eg[sc_] * s_rk[sc_];
#pragma unroll
        for (int e = 0; e < 16; ++e) dT[e] *= fr;
    }
    if (wP) {
#pragma unroll
        for (int s = 0; s < VS; ++s)
            dP = mfma32(lds_row8<PV>(tDO, 32 * tm + c, 16 * s + 8 * hh), lds_row8<PV>(tU, 32 * half + c, 16 * s + 8 * hh), dP);
    }
    lds_barrier();                                            // S0 and dS are dead: stage B loads reuse their space
    intra_load_tile<K>((lds_u32x4 *)(L + oQ), p.q + (int64_t)start * p.qst + (int64_t)hk * p.qsh, 2u * (uint32_t)p.qst,
                       len, wave, lane, NW);
    intra_load_tile<V>((lds_u32x4 *)(L + oVv), p.v + (int64_t)start * p.vst + (int64_t)h * p.vsh, 2u * (uint32_t)p.vst,
                       len, wave, lane, NW);
    intra_load_tile<64>((lds_u32x4 *)(L + oT), w.TB + chh * (64 * 64 / 8), 128u, 64, wave, lane, NW);
    vm_wait<0>();
    lds_barrier();
    // With several rounds of items, the item R = (CUs) on from this one (blocks R apart share an
    // XCD; the next round runs it there) has its S0 and dS cache lines touched now, one dword
    // per 128-byte line into a never-read LDS slot, so that its stage-A loads find them in the
    // L2 or the Infinity Cache.  GL: the item's next value head first (its stage-A wait is the
    // first to cover these loads), then the next item's first head; otherwise only the end of
    // the kernel waits for them.
    if (NW == 8) {
        int64_t nchh = -1;
        if (j + 1 < NH) {
            nchh = chh + 1;
        } else {
            const int R = p.intra_grid / 3, nb = (int)blockIdx.x + R;
            if ((int)gridDim.x > R && nb < (int)gridDim.x && nb / (GL ? p.HK : p.HV) < total)
                nchh = GL ? (int64_t)(nb / p.HK) * p.HV + (int64_t)(nb % p.HK) * G : (int64_t)nb;
        }
        if (nchh >= 0) {
            const i32x4 rS = make_rsrc(w.CK + nchh * K * V, (uint32_t)(K * V * 4));
            const i32x4 rD = make_rsrc(w.DSN + nchh * K * V, (uint32_t)(K * V * 4));
#pragma unroll
            for (int j = 0; j < K * V * 4 / 128 / (64 * NW); ++j) {
                const uint32_t off = (uint32_t)(tid + 64 * NW * j) * 128u;
                b2l_dword(rS, (lds_float *)(pf_sink + 64 * wave), off);
                b2l_dword(rD, (lds_float *)(pf_sink + 64 * wave), off);
            }
        }
    }
    // ---- B0: the output's state term of dgam: scale r_q rowdot(q, 2^gam dO S0^T) (dq^ holds
    // that term of this head and, with GL, the earlier heads' sum, whose row dot is qprev)
    {
        float prod[16] = {};
#pragma unroll
        for (int i = 0; i < IK; ++i) {
            float xq_[16];
            acc_elems<PK>(L + oQ, 32 * tm, 32 * ctile(i), lane, xq_);
#pragma unroll
            for (int e = 0; e < 16; ++e) prod[e] += dQ[i][e] * xq_[e];
        }
        {
            const float r = rowsum32(prod, lane) - qprev;
            const int e = c >> 1, row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
            if ((c & 1) == 0) part[QX][pw][row] = r * p.scale * s_rq[row];
        }
    }
    // ---- B2: P = M o (q^ k^T) for tile (tm, half); dP o P sums; R = M o dP r_k,s and R2 = M o dP scale r_q,t
    if (wP) {
        f32x16 qk = {};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qk = mfma32(lds_row8<PK>(tQ, 32 * tm + c, 16 * s + 8 * hh), lds_row8<PK>(tK, 32 * half + c, 16 * s + 8 * hh), qk);
        const int sI = 32 * half + c;
        const float gs = s_gam[sI], rs = s_rk[sI];
        f32x16 R, R2;
        float colsum = 0.f, ppv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int t = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
            const float m = exp2_hw(sI <= t ? s_gam[t] - gs : kNegInf);
            const float pv = p.scale * s_rq[t] * rs * m * qk[e];
            const float pp = dP[e] * pv;
            colsum += pp;
            ppv[e] = pp;
            R[e] = m * dP[e] * rs;
            R2[e] = m * dP[e] * p.scale * s_rq[t];
        }
        {
            const float r = rowsum32(ppv, lane);
            const int e = c >> 1;
            if ((c & 1) == 0) part[PPR_][half][32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3)] = r;
        }
        colsum += __shfl_xor(colsum, 32, 64);
        if (hh == 0) part[PPC][tm][sI] = colsum;
        store_tile_bf16<8>(L + oR, R, 32 * tm, 32 * half, lane);
        store_tile_bf16<8>(L + oR2, R2, 32 * tm, 32 * half, lane);
    }
    // ---- B3: dT's second term dU (diag(beta) V)^T; dT published in bf16
    if (wT) {
        f32x16 a = {};
#pragma unroll
        for (int s = 0; s < VS; ++s)
            a = mfma32(lds_row8<PV>(tDU, 32 * tm + c, 16 * s + 8 * hh), lds_row8<PV>(tV, 32 * half + c, 16 * s + 8 * hh), a);
        const float bs = s_b[32 * half + c];
#pragma unroll
        for (int e = 0; e < 16; ++e) dT[e] += a[e] * bs;
        store_tile_bf16<8>(L + oDT, dT, 32 * tm, 32 * half, lane);
    }
    // ---- B4: X2 = T^T dU (rows s of tile tm): dv = diag(beta) X2 and rowdot(X2, v) into dbeta
    {
        float prod[16] = {};
#pragma unroll
        for (int i = 0; i < IV; ++i) {
            const int vt = ctile(i);
            f32x16 a = {};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                a = mfma32(lds_tr32s<8, false>(tT, 16 * st, 32 * tm, lane), lds_tr32s<PV, false>(tDU, 16 * st, 32 * vt, lane), a);
            float xv[16];
            acc_elems<PV>(L + oVv, 32 * tm, 32 * vt, lane, xv);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
                prod[e] += a[e] * xv[e];
                if (row < len) dv_out[((int64_t)(start + row) * p.HV + h) * V + 32 * vt + c] = s_b[row] * a[e];
            }
        }
        {
            const float r = rowsum32(prod, lane);
            const int e = c >> 1;
            if ((c & 1) == 0) part[XV][pw][32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3)] = r;
        }
    }
    // ---- B5: X1 = T^T dW: dk^ += diag(f) X1 and df = r_k rowdot(X1, k)
    {
        float prod[16] = {};
#pragma unroll
        for (int i = 0; i < IK; ++i) {
            const int kt = ctile(i);
            f32x16 a = {};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                a = mfma32(lds_tr32s<8, false>(tT, 16 * st, 32 * tm, lane), lds_tr32s<PK, false>(tDW, 16 * st, 32 * kt, lane), a);
            float xk[16];
            acc_elems<PK>(L + oK, 32 * tm, 32 * kt, lane, xk);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
                prod[e] += a[e] * xk[e];
                dK[i][e] += s_b[row] * s_eg[row] * a[e];
            }
        }
        {
            const float r = rowsum32(prod, lane);
            const int e = c >> 1, row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
            if ((c & 1) == 0) part[DF][pw][row] = r * s_rk[row];
        }
    }
    lds_barrier();                                            // R, R2 and dT published
    // ---- B7, B8: dq^ += R k, dk^ += R2^T q
#pragma unroll
    for (int i = 0; i < IK; ++i) {
        const int kt = ctile(i);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            dQ[i] = mfma32(lds_row8<8>(tR, 32 * tm + c, 16 * st + 8 * hh), lds_tr32s<PK, false>(tK, 16 * st, 32 * kt, lane), dQ[i]);
            dK[i] = mfma32(lds_tr32s<8, false>(tR2, 16 * st, 32 * tm, lane), lds_tr32s<PK, false>(tQ, 16 * st, 32 * kt, lane), dK[i]);
        }
    }
    // one q/k head per value head, or the last head of the group: the row norms' chain rule is
    // applied here (dq_out set), and the row dots (q . dq^) it needs are taken while q is still
    // in LDS (dq^ is final)
    if (fuse_qk) {
        float prod[16] = {};
#pragma unroll
        for (int i = 0; i < IK; ++i) {
            float x[16];
            acc_elems<PK>(L + oQ, 32 * tm, 32 * ctile(i), lane, x);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                xq[i][e] = f2bf(x[e]);   // x is a bf16 value: exact
                prod[e] += dQ[i][e] * x[e];
            }
        }
        const float r = rowsum32(prod, lane);
        const int e = c >> 1;
        if (j == NH - 1) {
            if ((c & 1) == 0) part[QD][pw][32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3)] = r;
        } else {
            qprev = r;
        }
    }
    // ---- C1: Y = dT T^T, tile (tm, half); the Gram tile of k that C2 needs, tile (tm, half)
    f32x16 gk = {};
    {
        f32x16 y = {};
        if (wT) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
                y = mfma32(lds_row8<8>(tDT, 32 * tm + c, 16 * st + 8 * hh), lds_row8<8>(tT, 32 * half + c, 16 * st + 8 * hh), y);
        }
        if (wP) {
#pragma unroll
            for (int s = 0; s < KS; ++s)
                gk = mfma32(lds_row8<PK>(tK, 32 * tm + c, 16 * s + 8 * hh), lds_row8<PK>(tK, 32 * half + c, 16 * s + 8 * hh), gk);
        }
        lds_barrier();                                        // q, v, R and R2 are dead: Y, Z, Z3 reuse them
        if (wT) store_tile_bf16<8>(L + oY, y, 32 * tm, 32 * half, lane);
    }
    lds_barrier();
    // ---- C2: dA = -T^T Y (strictly lower), tile (rows a of tile tm, columns b of tile half), with
    // the Gram tile of k: A = beta_a E r_a r_b (k_a . k_b); dbeta, dgam sums; Z, Z3 = dGm r_b, dGm r_a.
    // Both wave groups form dA; the one with the Gram tile takes the sums, the other Z and Z3.
    {
        f32x16 da = {};
#pragma unroll
        for (int st = 0; st < 4; ++st)
            da = mfma32(lds_tr32s<8, false>(tT, 16 * st, 32 * tm, lane), lds_tr32s<8, false>(tY, 16 * st, 32 * half, lane), da);
        const int b = 32 * half + c;
        const float gb = s_gam[b], rb = s_rk[b];
        if (wP) {
            float colsum = 0.f, v1[16], v2[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int a = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
                const float E = exp2_hw(b < a ? s_gam[a] - gb : kNegInf);
                const float dam = b < a ? -da[e] : 0.f;
                const float ghat = s_rk[a] * rb * gk[e];
                const float aA = dam * s_b[a] * E * ghat;
                colsum += aA;
                v1[e] = aA;
                v2[e] = dam * E * ghat;
            }
            {
                const float r1 = rowsum32(v1, lane), r2 = rowsum32(v2, lane);
                const int e = c >> 1, a = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
                if ((c & 1) == 0) {
                    part[AAR][half][a] = r1;
                    part[DAEG][half][a] = r2;
                }
            }
            colsum += __shfl_xor(colsum, 32, 64);
            if (hh == 0) part[AAC][tm][b] = colsum;
        }
        if (wT) {
            f32x16 Z, Z3;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int a = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
                const float E = exp2_hw(b < a ? s_gam[a] - gb : kNegInf);
                const float dam = b < a ? -da[e] : 0.f;
                const float dgm = dam * s_b[a] * E;
                Z[e] = dgm * rb;
                Z3[e] = dgm * s_rk[a];
            }
            store_tile_bf16<8>(L + oZ, Z, 32 * tm, 32 * half, lane);
            store_tile_bf16<8>(L + oZ3, Z3, 32 * tm, 32 * half, lane);
        }
    }
    lds_barrier();
    // ---- C3: dk^ += Z k + Z3^T k; the q^ and k^ gradients out
#pragma unroll
    for (int i = 0; i < IK; ++i) {
        const int kt = ctile(i);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bf16x8 kb = lds_tr32s<PK, false>(tK, 16 * st, 32 * kt, lane);
            dK[i] = mfma32(lds_row8<8>(tZ, 32 * tm + c, 16 * st + 8 * hh), kb, dK[i]);
            dK[i] = mfma32(lds_tr32s<8, false>(tZ3, 16 * st, 32 * tm, lane), kb, dK[i]);
        }
        if (!fuse_qk) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
                if (row < len) {
                    const int64_t at = ((int64_t)(start + row) * p.HV + h) * K + 32 * kt + c;
                    w.DQH[at] = dQ[i][e];
                    w.DKH[at] = dK[i][e];
                }
            }
        }
    }
    if (fuse_qk && j == NH - 1) {
        float prod[16] = {};
#pragma unroll
        for (int i = 0; i < IK; ++i) {
            float xk[16];
            acc_elems<PK>(L + oK, 32 * tm, 32 * ctile(i), lane, xk);
#pragma unroll
            for (int e = 0; e < 16; ++e) prod[e] += dK[i][e] * xk[e];
        }
        const float r = rowsum32(prod, lane);
        const int e = c >> 1;
        if ((c & 1) == 0) part[KD][pw][32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3)] = r;
    }
    lds_barrier();                                            // every partial sum written
    // a per-token sum over the column tiles (wsum: the K- and V-wide results' partials, one
    // per wave pair) or over the two 32-token tiles (psum: the 64 x 64 ones)
    auto wsum = [&](int x, int t) {
        float r = part[x][0][t];
#pragma unroll
        for (int j = 1; j < 2 * NQ; ++j) r += part[x][j][t];
        return r;
    };
    auto psum = [&](int x, int t) { return part[x][0][t] + part[x][1][t]; };
    if (fuse_qk && j == NH - 1) {
        // dx = r dx^ - r^3 (x . dx^) x (times scale for q; r = 1 without the norm): q from the
        // registers taken above, k rows from LDS
        float rq[16], rk[16], cq[16], ck[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
            rq[e] = s_rq[row];
            rk[e] = s_rk[row];
            cq[e] = p.l2norm ? rq[e] * rq[e] * rq[e] * wsum(QD, row) : 0.f;
            ck[e] = p.l2norm ? rk[e] * rk[e] * rk[e] * wsum(KD, row) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < IK; ++i) {
            const int col = 32 * ctile(i) + c;
            float xks[16];
            acc_elems<PK>(L + oK, 32 * tm, 32 * ctile(i), lane, xks);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * tm + 8 * (e >> 2) + 4 * hh + (e & 3);
                if (row < len) {
                    const float xk = xks[e];
                    const int64_t at = ((int64_t)(start + row) * p.HK + hk) * K + col;
                    dq_out[at] = p.scale * (rq[e] * dQ[i][e] - cq[e] * bf2f(xq[i][e]));
                    dk_out[at] = rk[e] * dK[i][e] - ck[e] * xk;
                }
            }
        }
    }
    // ---- per token: dbeta and dgam, then dg by the reverse cumulative sum within the chunk
    if (tid < 64) {
        const int t = tid;
        const float df = wsum(DF, t);
        const float f = s_b[t] * s_eg[t];
        const float db = wsum(XV, t) + df * s_eg[t] + part[DAEG][0][t] + part[DAEG][1][t];
        const float F = wsum(KX, t);
        float dgam = df * f + psum(AAR, t) - psum(AAC, t) + psum(PPR_, t) - psum(PPC, t) + wsum(QX, t) - F;
        // the last token also carries sum F and 2^gam_n <dS, S0>
        float Fs = t < len ? F : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) Fs += __shfl_xor(Fs, off, 64);
        if (t == len - 1) {
            float sd = sdot[0];
#pragma unroll
            for (int j = 1; j < NW; ++j) sd += sdot[j];
            dgam += Fs + exp2_hw(s_gam[t]) * sd;
        }
        if (t < len) db_out[(int64_t)(start + t) * p.HV + h] = db;
        // dg: the reverse cumulative sum of dgam within the chunk (zeros past its end), by a
        // suffix scan across the wave
        float acc = t < len ? dgam : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(acc, off, 64);
            if (t + off < 64) acc += y;
        }
        if (t < len) dg_out[(int64_t)(start + t) * p.HV + h] = acc;
    }
    if (j + 1 < NH) lds_barrier();   // this head's sums and scalars are read before the next head's
    }
    if (NW == 8) vm_wait<0>();   // the touches land in LDS: done before the workgroup ends
}

// dq and dk from the per-value-head gradients of q^ and k^: the sum over each head group
// (fixed order), then through the row norms (q^ = scale r_q q, k^ = r_k k,
// r = 1 / sqrt(sum x^2 + 1e-6)): dx = r dx^ - r^3 (x . dx^) x (times scale for q).  K / 8
// lanes per (token, q/k head) row, 8 elements each.
template <int K>
__global__ __launch_bounds__(256) void k_bwd_qk(Prob p, const Ws w, float *dq, float *dk)
{
    constexpr int LPR = K / 8, RPB = 256 / LPR;
    if (w.hdr[0] != LA_DEVICE_OK) return;                                  // malformed cu_seqlens: write nothing
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;    // token * HK + hk
    const int piece = threadIdx.x % LPR;
    const bool live = row < p.T * p.HK;
    const int64_t t = live ? row / p.HK : 0;
    const int hk = live ? (int)(row % p.HK) : 0;
    const int G = p.HV / p.HK;
    float gq[8] = {}, gk[8] = {}, xq[8], xk[8];
    if (live) {
        const float4 *a = reinterpret_cast<const float4 *>(w.DQH + ((t * p.HV + hk * G) * K + 8 * piece));
        const float4 *b = reinterpret_cast<const float4 *>(w.DKH + ((t * p.HV + hk * G) * K + 8 * piece));
        for (int j = 0; j < G; ++j) {
            const float4 a0 = a[j * (K / 4)], a1 = a[j * (K / 4) + 1], b0 = b[j * (K / 4)], b1 = b[j * (K / 4) + 1];
            gq[0] += a0.x; gq[1] += a0.y; gq[2] += a0.z; gq[3] += a0.w;
            gq[4] += a1.x; gq[5] += a1.y; gq[6] += a1.z; gq[7] += a1.w;
            gk[0] += b0.x; gk[1] += b0.y; gk[2] += b0.z; gk[3] += b0.w;
            gk[4] += b1.x; gk[5] += b1.y; gk[6] += b1.z; gk[7] += b1.w;
        }
        const bf16x8 q8 = *reinterpret_cast<const bf16x8 *>(p.q + t * p.qst + (int64_t)hk * p.qsh + 8 * piece);
        const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(p.k + t * p.kst + (int64_t)hk * p.ksh + 8 * piece);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            xq[e] = bf2f(q8[e]);
            xk[e] = bf2f(k8[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xq[e] = xk[e] = 0.f;
    }
    float sq = 0.f, sk = 0.f, dqx = 0.f, dkx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sq = fmaf(xq[e], xq[e], sq);
        sk = fmaf(xk[e], xk[e], sk);
        dqx = fmaf(xq[e], gq[e], dqx);
        dkx = fmaf(xk[e], gk[e], dkx);
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) {
        sq += __shfl_xor(sq, off, 64);
        sk += __shfl_xor(sk, off, 64);
        dqx += __shfl_xor(dqx, off, 64);
        dkx += __shfl_xor(dkx, off, 64);
    }
    if (!live) return;
    const float rq = p.l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f, rk = p.l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
    const float cq = p.l2norm ? rq * rq * rq * dqx : 0.f, ck = p.l2norm ? rk * rk * rk * dkx : 0.f;
    float oq[8], ok[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        oq[e] = p.scale * (rq * gq[e] - cq * xq[e]);
        ok[e] = rk * gk[e] - ck * xk[e];
    }
    float4 *dq4 = reinterpret_cast<float4 *>(dq + (t * p.HK + hk) * K + 8 * piece);
    float4 *dk4 = reinterpret_cast<float4 *>(dk + (t * p.HK + hk) * K + 8 * piece);
    dq4[0] = make_float4(oq[0], oq[1], oq[2], oq[3]);
    dq4[1] = make_float4(oq[4], oq[5], oq[6], oq[7]);
    dk4[0] = make_float4(ok[0], ok[1], ok[2], ok[3]);
    dk4[1] = make_float4(ok[4], ok[5], ok[6], ok[7]);
}

// The reverse pass with two 32-column tiles per workgroup: for batches whose one-tile
// workgroups (one per CU) would need more than one round of the CUs.  Its chunk step runs
// both tiles in about the time of one (dense batch of 8 x 4096 tokens, HV = 16: 363 ->
// 223 us; 32 spans of 8192 tokens: 1807 -> 1094 us; the ragged batch with a 65,536-token
// sequence at H = 32: whole backward 18.4 -> 17.9 ms).
static bool bwd_wide(int64_t blocks, const Prob &p)
{
    const int64_t cus = p.intra_grid / 3;
    return (p.V / 32) % 2 == 0 && blocks > cus;
}

hipError_t run_backward(const Prob &p, const Ws &w_in, const BwdArgs &a, hipStream_t s, const LaunchHook *hook)
{
    // the chunk-start states: the caller's (the forward's fp32 series every 64 tokens, the
    // same rows the forward run again would write), or the workspace's
    Ws w = w_in;
    if (a.chunk_states) w.CK = const_cast<float *>(a.chunk_states);
    auto before = [&](int id) { if (hook) hook->before(id, s, hook->ctx); };
    auto after = [&](int id) { if (hook) hook->after(id, s, hook->ctx); };
    if (p.N == 0) return hipSuccess;
    if (p.N > 64) {
        before(LA_KERNEL_SCHED);
        hipLaunchKernelGGL(k_sched, dim3(1), dim3(1024), 0, s, p, w);
        after(LA_KERNEL_SCHED);
    }
    const int64_t items = (int64_t)p.max_chunks * p.HV;
    const int grid = (int)(items < p.intra_grid ? items : p.intra_grid);
    const unsigned inter_blocks = (unsigned)((int64_t)p.N * p.HV * (p.V / 32));
    const unsigned qk_blocks = (unsigned)((p.T * p.HK + 256 / (p.K / 8) - 1) / (256 / (p.K / 8)));
    // one value head per q/k head: no head-group sums, the intra pass writes dq and dk itself
    const bool fuse_qk = p.HV == p.HK;
    // K = V = 128 with head groups: one workgroup takes the G value heads of a (chunk, q/k
    // head) one after another and sums dq^ and dk^ in registers, so that the per-value-head
    // fp32 gradients never go through memory and k_bwd_qk does not run (dense batch of 8 x 4096
    // tokens, HK = 4, HV = 16: intra pass with k_bwd_qk 897 -> 769 us), unless its coarser
    // items would cost the CUs more than 1.3 times the rounds of single-head items (what the
    // saved head-group pass and gradient traffic cost, about 0.3 of a round per round there)
    const int64_t cus = p.intra_grid / 3, G = p.HV / p.HK;
    const int64_t items_g = (int64_t)p.max_chunks * p.HK;
    const bool group_loop = G > 1 && cus > 0 && 10 * G * ((items_g + cus - 1) / cus) <= 13 * ((items + cus - 1) / cus);
    // the forward again, with the state at every chunk start (fp32, indexed by chunk id)
    Prob pf = p;
    pf.ck_every = kChunk;
    pf.ck_fp32 = 1;
    pf.ck_quad = 1;
    // the intra pass reads the chunk-start states in the layout they come in
    Prob pb = p;
    pb.ck_quad = a.chunk_states ? 0 : 1;
    pf.ck = w.CK;
    pf.ck_cap = p.max_chunks;
    pf.o = nullptr;
    pf.sT = nullptr;
// waves of the backward's intra workgroup: 8 where both K and V split into four 32-column tiles
#define BWD_NW(KK, VV) ((KK) % 128 == 0 && (VV) % 128 == 0 ? 8 : 4)
#define LA_BWD(KK, VV)                                                                                         \
    if (p.K == KK && p.V == VV) {                                                                              \
        before(LA_KERNEL_INTRA);                                                                               \
        if (grid > 0)                                                                                          \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_intra<KK, VV, true, false, 2>), dim3(grid), dim3(256), 0, s, p, w); \
        after(LA_KERNEL_INTRA);                                                                                \
        before(LA_KERNEL_INTER);                                                                               \
        if (!a.chunk_states && (VV / 32) % 2 == 0 && inter_blocks > (unsigned)(p.intra_grid / 3))              \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_states_wide<KK, VV>), dim3(inter_blocks / 2), dim3(384), 0, s, \
                               pf, w);                                                                         \
        else if (!a.chunk_states)                                                                              \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_inter_states<KK, VV>), dim3(inter_blocks), dim3(256), 0, s, pf, w); \
        if (bwd_wide(inter_blocks, p))                                                                         \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_bwd_inter<KK, VV, true, 2>), dim3(inter_blocks / 2), dim3(384), 0, s, \
                               p, w, a.d_out, a.d_final, a.d_init);                                            \
        else                                                                                                   \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_bwd_inter<KK, VV, true>), dim3(inter_blocks), dim3(256), 0, s, p, w, \
                               a.d_out, a.d_final, a.d_init);                                                  \
        after(LA_KERNEL_INTER);                                                                                \
        before(LA_KERNEL_BWD_INTRA);                                                                           \
        bool looped = false;                                                                                   \
        if constexpr (BWD_NW(KK, VV) == 8) {                                                                   \
            if (group_loop && items_g > 0) {                                                                   \
                hipLaunchKernelGGL(HIP_KERNEL_NAME(k_bwd_intra<KK, VV, 8, true>), dim3((unsigned)items_g),       \
                                   dim3(512), 0, s, pb, w, a.d_out, a.dv, a.dg, a.dbeta, a.dq, a.dk);         \
                looped = true;                                                                                 \
            }                                                                                                  \
        }                                                                                                      \
        if (!looped && items > 0)                                                                              \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_bwd_intra<KK, VV, BWD_NW(KK, VV), false>), dim3((unsigned)items), \
                               dim3(64 * BWD_NW(KK, VV)), 0, s, pb, w, a.d_out, a.dv, a.dg, a.dbeta,           \
                               fuse_qk ? a.dq : nullptr, fuse_qk ? a.dk : nullptr);                           \
        if (!fuse_qk && !looped && qk_blocks > 0)                                                              \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_bwd_qk<KK>), dim3(qk_blocks), dim3(256), 0, s, p, w, a.dq, a.dk); \
        after(LA_KERNEL_BWD_INTRA);                                                                            \
        return hipGetLastError();                                                                              \
    }
    LA_BWD(64, 64)
    LA_BWD(64, 128)
    LA_BWD(128, 64)
    LA_BWD(128, 128)
#undef LA_BWD
#undef BWD_NW
    return hipErrorInvalidValue;
}

hipError_t run_summary_bwd(const Prob &p, const Ws &w, const __bf16 *d_out, const float *d_end, float *d_start,
                           hipStream_t s, const LaunchHook *hook)
{
    auto before = [&](int id) { if (hook) hook->before(id, s, hook->ctx); };
    auto after = [&](int id) { if (hook) hook->after(id, s, hook->ctx); };
    if (p.N == 0) return hipSuccess;
    if (p.N > 64) {
        before(LA_KERNEL_SCHED);
        hipLaunchKernelGGL(k_sched, dim3(1), dim3(1024), 0, s, p, w);
        after(LA_KERNEL_SCHED);
    }
    const int64_t items = (int64_t)p.max_chunks * p.HV;
    const int grid = (int)(items < p.intra_grid ? items : p.intra_grid);
    const unsigned blocks = (unsigned)((int64_t)p.N * p.HV * (p.V / 32));
#define LA_SBWD(KK, VV)                                                                                  \
    if (p.K == KK && p.V == VV) {                                                                        \
        before(LA_KERNEL_INTRA);                                                                         \
        if (grid > 0)                                                                                    \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_intra<KK, VV, true, false, 1>), dim3(grid), dim3(256), 0, s, p, w); \
        after(LA_KERNEL_INTRA);                                                                          \
        before(LA_KERNEL_INTER);                                                                         \
        if (bwd_wide(blocks, p))                                                                         \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_bwd_inter<KK, VV, false, 2>), dim3(blocks / 2), dim3(384), 0, s, p, w, \
                               d_out, d_end, d_start);                                                   \
        else                                                                                             \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_bwd_inter<KK, VV, false>), dim3(blocks), dim3(256), 0, s, p, w, \
                               d_out, d_end, d_start);                                                   \
        after(LA_KERNEL_INTER);                                                                          \
        return hipGetLastError();                                                                        \
    }
    LA_SBWD(64, 64)
    LA_SBWD(64, 128)
    LA_SBWD(128, 64)
    LA_SBWD(128, 128)
#undef LA_SBWD
    return hipErrorInvalidValue;
}

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
