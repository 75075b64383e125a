"""A numpy model of the chunked method the HIP kernels use (test infrastructure).

The chunked evaluation of the Gated DeltaNet recurrence (the cuDNN "Linear
Attention" page describes the op as evaluated in chunks; the cudnn-frontend PR
"Further reduce FROST LA CPU overhead + fully support all L2norm, beta, gate
fusion" names its steps: a chunk-local cumulative gate, the intra-chunk UT/WY
solve that returns w, u and A, and the inter-chunk state pass).  Per (sequence,
value head) and per chunk of n <= 64 tokens with start state S0 (K x V), with
k^ = r_k k, q^ = scale r_q q and gam the chunk-local inclusive cumsum of g:

    A[t, s] = beta_t exp(gam_t - gam_s) (k^_t . k^_s)      for s < t, else 0
    T       = (I + A)^-1                                   (unit lower triangular)
    W       = T diag(beta exp(gam)) K^,   U~ = T diag(beta) V
    U       = U~ - W S0
    O       = diag(exp(gam)) Q^ S0 + (Mask o Q^ K^T) U,   Mask[t, s] = exp(gam_t - gam_s), s <= t
    S_n     = exp(gam_n) S0 + K^T diag(exp(gam_n - gam)) U

Unrolling the token recurrence over a chunk gives these formulas exactly, so in
fp64 this model must equal the token-by-token oracle to rounding (the test pins
it at 1e-12).  `Rounding` selects where the model rounds to bf16 or fp32, at
the points where the kernels do, so that the error of a kernel design can be
predicted before it runs.  The model shares nothing with the HIP path: it is
written from the formulas above.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

CHUNK = 64


def bf16(x) -> np.ndarray:
    """Round to bf16 (round to nearest, ties to even) through fp32; returned as fp64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def f16_tiles(x: np.ndarray, tile: int = 32) -> np.ndarray:
    """x [..., n, m] (fp32 values) rounded to fp16 per tile x tile block, each block scaled
    first by the power of two 2^(15 - E), E the exponent with max|block| in [2^(E-1), 2^E),
    and scaled back exactly afterwards (all-zero blocks stay zero)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    n, m = x.shape[-2:]
    for r0 in range(0, n, tile):
        for c0 in range(0, m, tile):
            blk = x[..., r0:r0 + tile, c0:c0 + tile]
            amax = np.max(np.abs(blk), axis=(-2, -1), keepdims=True)
            e = np.frexp(amax)[1]
            scaled = np.ldexp(blk, 15 - e).astype(np.float32).astype(np.float16)
            out[..., r0:r0 + tile, c0:c0 + tile] = np.ldexp(scaled.astype(np.float64), e - 15)
    return out


def unit_lower_inverse(A: np.ndarray) -> np.ndarray:
    """(I + A)^-1 for strictly lower-triangular A ([..., n, n]) by forward substitution,
    column by column: x_i = e_i - sum_{k<i} A[i, k] x_k, one row at a time."""
    n = A.shape[-1]
    T = np.zeros_like(A)
    for i in range(n):
        T[..., i, i] = 1.0
        if i:
            T[..., i, :i] = -np.einsum("...k,...kj->...j", A[..., i, :i], T[..., :i, :i])
    return T


@dataclasses.dataclass
class Rounding:
    """Where the model rounds.  exact: none at all (fp64 throughout).  Otherwise the
    kernel design: W and P^T in bf16, T diag(beta) as a bf16 hi/lo pair (so U~ is
    about fp32), S rounded to bf16 as the operand of W S and Q S, diag(d) U rounded to
    bf16 as the operand of the state update, U rounded to bf16 as the operand of P U,
    states kept in fp32, o rounded to bf16.  ut_bf16 instead rounds U~ itself to bf16
    (the plain all-bf16 design); ut_f16 rounds the about-fp32 U~ to fp16 after scaling
    each 32 x 32 tile (32 tokens, 32 value columns) by a power of two that puts its
    largest magnitude in [2^14, 2^15) (the kernels' hand-over format)."""
    exact: bool = True
    ut_bf16: bool = False
    ut_f16: bool = False

    def r16(self, x):
        return x if self.exact else bf16(x)

    def r32(self, x):
        return x if self.exact else f32(x)


EXACT = Rounding(exact=True)
KERNEL = Rounding(exact=False)
ALL_BF16 = Rounding(exact=False, ut_bf16=True)
KERNEL_F16 = Rounding(exact=False, ut_f16=True)


def _masked_exp(gam: np.ndarray, strict: bool) -> np.ndarray:
    """exp(gam_t - gam_s) for s < t (strict) or s <= t, zero elsewhere; [..., n, n]."""
    n = gam.shape[-1]
    keep = np.tril(np.ones((n, n), dtype=bool), -1 if strict else 0)
    diff = gam[..., :, None] - gam[..., None, :]
    return np.exp(np.where(keep, diff, -np.inf))


def chunked_sequence(q, k, v, g, beta, S0, scale: float, l2norm: bool, rounding: Rounding = EXACT,
                     chunk: int = CHUNK) -> Tuple[Optional[np.ndarray], np.ndarray]:
    """One sequence, all value heads at once.

    q, k: [L, H, K] (q may be None: no output), v: [L, H, V], g, beta: [L, H], S0:
    [H, K, V] (fp64 values).  The heads here are value heads: grouped q/k heads are
    expanded by the caller.  Returns o [L, H, V] (or None) and the final state."""
    L, H, _ = k.shape
    V = v.shape[2]
    rnd = rounding
    rk = 1.0 / np.sqrt(np.sum(k * k, axis=2) + 1e-6) if l2norm else np.ones((L, H))
    rq = (1.0 / np.sqrt(np.sum(q * q, axis=2) + 1e-6) if l2norm else np.ones((L, H))) if q is not None else None
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((L, H, V)) if q is not None else None
    for c0 in range(0, L, chunk):
        c1 = min(c0 + chunk, L)
        # heads first: [H, n, .]
        Kc = np.transpose(k[c0:c1], (1, 0, 2))
        Vc = np.transpose(v[c0:c1], (1, 0, 2))
        b = beta[c0:c1].T
        gam = np.cumsum(g[c0:c1].T, axis=1)
        r = rk[c0:c1].T
        Kh = r[:, :, None] * Kc
        A = b[:, :, None] * _masked_exp(gam, strict=True) * (Kh @ np.transpose(Kh, (0, 2, 1)))
        T = unit_lower_inverse(A)
        # W = T diag(beta e^gam r_k) K (raw K), U~ = T diag(beta) V
        Tw = rnd.r16(T * (b * np.exp(gam) * r)[:, None, :])
        W = rnd.r16(Tw @ Kc)
        TB = T * b[:, None, :]
        if rnd.exact:
            Ut = TB @ Vc
        elif rnd.ut_bf16:
            Ut = bf16(TB @ Vc)
        else:
            hi = bf16(TB)
            lo = bf16(TB - hi)
            Ut = f32(hi @ Vc + lo @ Vc)
            if rnd.ut_f16:
                Ut = f16_tiles(Ut)
        Sb = rnd.r16(S)
        U = rnd.r32(Ut - W @ Sb)
        gn = gam[:, -1]
        d = np.exp(gn[:, None] - gam) * r
        if q is not None:
            Qc = np.transpose(q[c0:c1], (1, 0, 2))
            sq = scale * rq[c0:c1].T * np.exp(gam)
            P = rnd.r16(scale * rq[c0:c1].T[:, :, None] * r[:, None, :] * _masked_exp(gam, strict=False)
                        * (Qc @ np.transpose(Kc, (0, 2, 1))))
            oc = sq[:, :, None] * (Qc @ Sb) + P @ rnd.r16(U)
            o[c0:c1] = np.transpose(rnd.r16(oc), (1, 0, 2))
        S = rnd.r32(np.exp(gn)[:, None, None] * S + np.transpose(Kc, (0, 2, 1)) @ rnd.r16(d[:, :, None] * U))
    return o, S


def chunked_forward(problem, rounding: Rounding = EXACT, scale: Optional[float] = None):
    """Every sequence of a workloads.Problem: o [T, HV, V] (None for a summary problem)
    and final states [N, HV, K, V], from the problem's initial state (or zeros)."""
    p = problem
    k = p.k.float().double().numpy()
    v = p.v.float().double().numpy()
    q = p.q.float().double().numpy() if p.q is not None else None
    g = p.g.double().numpy()
    beta = p.beta.double().numpy()
    HK, HV = k.shape[1], v.shape[1]
    K, V = k.shape[2], v.shape[2]
    rep = np.arange(HV) // (HV // HK)
    sc = K ** -0.5 if scale is None else scale
    cu = p.cu_seqlens.tolist()
    N = len(cu) - 1
    o = np.zeros((cu[-1], HV, V)) if q is not None else None
    fin = np.zeros((N, HV, K, V))
    for n in range(N):
        a, e = cu[n], cu[n + 1]
        S0 = p.state[n].double().numpy() if p.state is not None else np.zeros((HV, K, V))
        if e == a:
            fin[n] = S0
            continue
        on, fin[n] = chunked_sequence(None if q is None else q[a:e][:, rep], k[a:e][:, rep], v[a:e], g[a:e],
                                      beta[a:e], S0, sc, p.l2norm, rounding)
        if o is not None:
            o[a:e] = on
    return o, fin


def chunked_backward_sequence(q, k, v, g, beta, S0, dO, dS_final, scale: float, l2norm: bool,
                              rounding: Rounding = EXACT, chunk: int = CHUNK):
    """Gradients of one sequence (all value heads at once) by the chunked method: the
    forward above run again to get each chunk's start state, then the chunks in reverse
    with the end-state gradient dS carried from chunk to chunk,
        dU  = diag(exp(gam_n - gam)) K^ dS + P^T dO
        dS0 = exp(gam_n) dS + Q^T diag(exp(gam)) dO - W^T dU
    and, per chunk, the gradients of everything the forward formed from q, k, v, beta
    and gam (through P, W, U~, T = (I + A)^-1 with dA = -T^T dT T^T, and the decays),
    then through the chunk-local cumsum to g and through the row norms to q and k.
    Shapes as chunked_sequence, plus dO [L, H, V] and dS_final [H, K, V].  Returns dq, dk
    [L, H, K] (per value head; the caller sums a head group), dv [L, H, V], dg, dbeta
    [L, H] and the start-state gradient [H, K, V]."""
    L, H, K = k.shape
    V = v.shape[2]
    rnd = rounding
    rk = 1.0 / np.sqrt(np.sum(k * k, axis=2) + 1e-6) if l2norm else np.ones((L, H))
    rq = 1.0 / np.sqrt(np.sum(q * q, axis=2) + 1e-6) if l2norm else np.ones((L, H))
    tr = lambda x: np.transpose(x, (0, 2, 1))
    # forward again: every chunk's start state
    starts = []
    S = np.array(S0, dtype=np.float64)
    for c0 in range(0, L, chunk):
        starts.append(S)
        c1 = min(c0 + chunk, L)
        _, S = chunked_sequence(None, k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1], S, scale, l2norm, rounding,
                                chunk)
    dq = np.zeros((L, H, K))
    dk = np.zeros((L, H, K))
    dv = np.zeros((L, H, V))
    dg = np.zeros((L, H))
    db = np.zeros((L, H))
    dS = np.array(dS_final, dtype=np.float64)
    for ci in range(len(starts) - 1, -1, -1):
        c0 = ci * chunk
        c1 = min(c0 + chunk, L)
        S0c = starts[ci]
        Kc = np.transpose(k[c0:c1], (1, 0, 2))             # [H, n, K]
        Qc = np.transpose(q[c0:c1], (1, 0, 2))
        Vc = np.transpose(v[c0:c1], (1, 0, 2))
        dOc = np.transpose(dO[c0:c1], (1, 0, 2))
        b = beta[c0:c1].T
        gam = np.cumsum(g[c0:c1].T, axis=1)
        r, s_q = rk[c0:c1].T, rq[c0:c1].T
        Kh = r[:, :, None] * Kc
        Qh = scale * s_q[:, :, None] * Qc
        eg = np.exp(gam)
        gn = gam[:, -1]
        d = np.exp(gn[:, None] - gam)
        Eg = _masked_exp(gam, strict=True)
        G = Kh @ tr(Kh)
        A = b[:, :, None] * Eg * G
        T = unit_lower_inverse(A)
        f = b * eg
        W = T @ (f[:, :, None] * Kh)
        U = T @ (b[:, :, None] * Vc) - W @ S0c
        M = _masked_exp(gam, strict=False)
        P = M * (Qh @ tr(Kh))
        # the carried gradient (B(.): where the kernels round an MFMA operand to bf16)
        B = rnd.r16
        if not rnd.exact:
            Tw = B(T * (f * r)[:, None, :])
            W = B(Tw @ Kc)                                  # as the forward's intra pass forms it
            TB = T * b[:, None, :]
            hi = bf16(TB)
            Ut = f32(hi @ Vc + bf16(TB - hi) @ Vc)
            if rnd.ut_f16:
                Ut = f16_tiles(Ut)
            U = f32(Ut - W @ B(S0c))
        dU = d[:, :, None] * (Kh @ B(dS)) + B(tr(P)) @ dOc
        dS_prev = (np.exp(gn)[:, None, None] * dS + tr(Qc) @ B(scale * (s_q * eg)[:, :, None] * dOc)
                   - tr(W) @ B(dU))
        # q, k through P and the output's state term; k through the state update
        dP = M * (dOc @ tr(B(U)))
        dQh = eg[:, :, None] * (dOc @ tr(B(S0c))) + B(dP * r[:, None, :]) @ Kc
        UdS = B(U) @ tr(B(dS))                              # [H, n, K]
        dKh = tr(B(dP * scale * s_q[:, :, None])) @ Qc + d[:, :, None] * UdS
        # W = T diag(f) K^ and U~ = T diag(beta) V
        Tb = B(T)
        dW = -(B(dU) @ tr(B(S0c)))
        X1 = tr(Tb) @ B(dW)
        X2 = tr(Tb) @ B(dU)
        dKh += f[:, :, None] * X1
        df = np.sum(X1 * Kh, axis=2)
        dVc = b[:, :, None] * X2
        dbc = np.sum(X2 * Vc, axis=2) + df * eg
        dgam = df * f
        dT = (B(dW) @ tr(Kc)) * (f * r)[:, None, :] + (B(dU) @ tr(Vc)) * b[:, None, :]
        dA = -(tr(Tb) @ B(B(dT) @ tr(Tb))) * np.tril(np.ones_like(A[0]), -1)
        dGm = dA * b[:, :, None] * Eg
        dKh += B(dGm * r[:, None, :]) @ Kc + B(tr(dGm) * r[:, None, :]) @ Kc
        dbc += np.sum(dA * Eg * G, axis=2)
        aA = dA * A
        dgam += np.sum(aA, axis=2) - np.sum(aA, axis=1)
        pP = (dOc @ tr(B(U))) * P                       # dP o P (zero outside the mask)
        dgam += np.sum(pP, axis=2) - np.sum(pP, axis=1)
        dgam += eg * np.sum((Qh @ B(S0c)) * dOc, axis=2)
        F = d * np.sum(Kh * UdS, axis=2)
        dgam -= F
        dgam[:, -1] += np.sum(F, axis=1) + np.exp(gn) * np.sum(dS * S0c, axis=(1, 2))
        # chunk-local cumsum, then the row norms
        dgc = np.cumsum(dgam[:, ::-1], axis=1)[:, ::-1]
        if l2norm:
            dKc = r[:, :, None] * dKh - (r ** 3 * np.sum(Kc * dKh, axis=2))[:, :, None] * Kc
            dQc = scale * (s_q[:, :, None] * dQh - (s_q ** 3 * np.sum(Qc * dQh, axis=2))[:, :, None] * Qc)
        else:
            dKc = dKh
            dQc = scale * dQh
        dq[c0:c1] = np.transpose(dQc, (1, 0, 2))
        dk[c0:c1] = np.transpose(dKc, (1, 0, 2))
        dv[c0:c1] = np.transpose(dVc, (1, 0, 2))
        dg[c0:c1] = dgc.T
        db[c0:c1] = dbc.T
        dS = dS_prev
    return dq, dk, dv, dg, db, dS


def chunked_backward(problem, d_o, d_final=None, rounding: Rounding = EXACT, scale: Optional[float] = None):
    """Gradients of a workloads.Problem's forward (plain gate and beta) for upstream
    gradients d_o [T, HV, V] and d_final [N, HV, K, V] (None: zeros), by the chunked
    method: dq, dk [T, HK, K] (summed over each head group), dv [T, HV, V], dg, dbeta
    [T, HV] and d_init [N, HV, K, V]."""
    p = problem
    k = p.k.float().double().numpy()
    v = p.v.float().double().numpy()
    q = p.q.float().double().numpy()
    g = p.g.double().numpy()
    beta = p.beta.double().numpy()
    HK, HV = k.shape[1], v.shape[1]
    K, V = k.shape[2], v.shape[2]
    G = HV // HK
    rep = np.arange(HV) // G
    sc = K ** -0.5 if scale is None else scale
    cu = p.cu_seqlens.tolist()
    N = len(cu) - 1
    T = cu[-1]
    d_o = np.asarray(d_o, dtype=np.float64)
    out = {"dq": np.zeros((T, HK, K)), "dk": np.zeros((T, HK, K)), "dv": np.zeros((T, HV, V)),
           "dg": np.zeros((T, HV)), "dbeta": np.zeros((T, HV)), "d_init": np.zeros((N, HV, K, V))}
    for n in range(N):
        a, e = cu[n], cu[n + 1]
        dF = np.zeros((HV, K, V)) if d_final is None else np.asarray(d_final[n], dtype=np.float64)
        if e == a:
            out["d_init"][n] = dF
            continue
        S0 = p.state[n].double().numpy() if p.state is not None else np.zeros((HV, K, V))
        dq, dk, dv, dg, db, di = chunked_backward_sequence(q[a:e][:, rep], k[a:e][:, rep], v[a:e], g[a:e],
                                                           beta[a:e], S0, d_o[a:e], dF, sc, p.l2norm, rounding)
        out["dq"][a:e] = dq.reshape(e - a, HK, G, K).sum(axis=2)
        out["dk"][a:e] = dk.reshape(e - a, HK, G, K).sum(axis=2)
        out["dv"][a:e] = dv
        out["dg"][a:e] = dg
        out["dbeta"][a:e] = db
        out["d_init"][n] = di
    return out
