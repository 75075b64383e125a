"""Seeded synthetic inputs for the Gated DeltaNet forward and span summary.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic, so both the fp64 oracle and the GPU path may use it.

The shapes and distributions follow the example call on the cuDNN
"Linear Attention" page (section "Example"): packed THD tensors q, k, v of
N(0, 1) values stored as bf16, a log-space gate g = -softplus(N(0, 1)) and
beta = sigmoid(N(0, 1)), both fp32 and laid out [T, heads], and int32
cu_seqlens.  Initial (start) states are fp32 N(0, 0.1^2).

Draw order is fixed so a seed always gives the same tensors:
lengths -> q -> k -> v -> g_raw -> beta_raw -> state.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

__all__ = ["Problem", "CONFIGS", "make_problem", "custom_problem", "config_lengths"]


@dataclasses.dataclass
class Problem:
    """One synthetic problem, all tensors on the CPU unless moved."""

    name: str
    cu_seqlens: torch.Tensor          # int32 [N + 1]
    q: Optional[torch.Tensor]         # bf16 [T, HK, K] (None for a summary)
    k: torch.Tensor                   # bf16 [T, HK, K]
    v: torch.Tensor                   # bf16 [T, HV, V]
    g: torch.Tensor                   # fp32 [T, HV], natural-log gate
    beta: torch.Tensor                # fp32 [T, HV]
    state: Optional[torch.Tensor]     # fp32 [N, HV, K, V] or None (zero start)
    l2norm: bool = True
    summary: bool = False
    # gate and beta transforms: with beta_sigmoid, `beta` holds bf16 logits; with a_log,
    # `g` holds the raw gate and g = -exp(a_log) softplus(g + dt_bias) per value head
    beta_sigmoid: bool = False
    a_log: Optional[torch.Tensor] = None     # fp32 [HV]
    dt_bias: Optional[torch.Tensor] = None   # fp32 [HV] or None
    # Gated Delta Product: k, v and beta have num_householder rows per token (update-major)
    num_householder: int = 1

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.numel()) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.k.shape[0]) // self.num_householder

    @property
    def num_qk_heads(self) -> int:
        return int(self.k.shape[1])

    @property
    def num_v_heads(self) -> int:
        return int(self.v.shape[1])

    @property
    def head_dim_k(self) -> int:
        return int(self.k.shape[2])

    @property
    def head_dim_v(self) -> int:
        return int(self.v.shape[2])

    def lengths(self) -> List[int]:
        cu = self.cu_seqlens.tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]

    def to(self, device) -> "Problem":
        def mv(x):
            return None if x is None else x.to(device)
        return dataclasses.replace(
            self, cu_seqlens=mv(self.cu_seqlens), q=mv(self.q), k=mv(self.k), v=mv(self.v),
            g=mv(self.g), beta=mv(self.beta), state=mv(self.state), a_log=mv(self.a_log),
            dt_bias=mv(self.dt_bias))


# The five workloads.  "lengths" is a list, or "ragged" for the case whose
# lengths are drawn from the generator.  Companion variants (slow decay: g/4096, beta/64) exist for
# 3 and 5, because under the plain gate the transition underflows to zero and
# the initial state barely reaches the output.
CONFIGS: Dict[int, dict] = {
    1: dict(name="tiny: T=256, N=1, H=2, K=V=64", lengths=[256], hk=2, hv=2, dk=64, dv=64,
            state=False, summary=False),
    2: dict(name="varlen: T=4096, N=3 (1000,1500,1596), H=16, K=V=128",
            lengths=[1000, 1500, 1596], hk=16, hv=16, dk=128, dv=128, state=False, summary=False),
    3: dict(name="dense batch: 8 x 4096, HK=4, HV=16, K=V=128, initial state",
            lengths=[4096] * 8, hk=4, hv=16, dk=128, dv=128, state=True, summary=False),
    4: dict(name="ragged long context: 64 x U[1,4096] + 65536, H=32, K=V=128",
            lengths="ragged", hk=32, hv=32, dk=128, dv=128, state=False, summary=False),
    5: dict(name="span summary: 32 x 8192, H=16, K=V=128, start state",
            lengths=[8192] * 32, hk=16, hv=16, dk=128, dv=128, state=True, summary=True),
}


def _ragged_lengths(gen: torch.Generator) -> List[int]:
    lens = torch.randint(1, 4097, (64,), generator=gen).tolist()
    lens[0] = 1          # a length-1 sequence
    lens[1] = 64         # exactly one chunk
    assert any(x % 64 for x in lens)
    return lens + [65536]


def config_lengths(cfg_id: int, seed: Optional[int] = None) -> List[int]:
    """Sequence lengths of a config (draws only the lengths)."""
    cfg = CONFIGS[cfg_id]
    if cfg["lengths"] == "ragged":
        gen = torch.Generator().manual_seed(cfg_id if seed is None else seed)
        return _ragged_lengths(gen)
    return list(cfg["lengths"])


def _draw(gen, lengths, hk, hv, dk, dv, with_state, with_q, device):
    T = int(sum(lengths))
    N = len(lengths)
    cu = torch.zeros(N + 1, dtype=torch.int64)
    if N:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    cu = cu.to(torch.int32)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)

    q = randn(T, hk, dk).to(torch.bfloat16)
    k = randn(T, hk, dk).to(torch.bfloat16)
    v = randn(T, hv, dv).to(torch.bfloat16)
    g = -torch.nn.functional.softplus(randn(T, hv))
    beta = torch.sigmoid(randn(T, hv))
    state = (0.1 * randn(N, hv, dk, dv)) if with_state else None
    if not with_q:
        q = None
    return cu, q, k, v, g, beta, state


def make_problem(cfg_id: int, companion: bool = False, seed: Optional[int] = None,
                 device: str = "cpu") -> Problem:
    """Inputs of config `cfg_id` (1..5).

    companion=True gives the slow-decay variant (g / 4096, beta / 64, seed
    100 + id) on which the transition and the initial state are far from zero.
    `device` is where the random numbers are drawn; the CPU is the default so
    the oracle and the GPU see the same tensors.
    """
    cfg = CONFIGS[cfg_id]
    if seed is None:
        seed = (100 + cfg_id) if companion else cfg_id
    gen = torch.Generator(device=device).manual_seed(seed)
    if cfg["lengths"] == "ragged":
        lengths = _ragged_lengths(torch.Generator().manual_seed(seed))
    else:
        lengths = list(cfg["lengths"])
    cu, q, k, v, g, beta, state = _draw(gen, lengths, cfg["hk"], cfg["hv"], cfg["dk"], cfg["dv"],
                                        cfg["state"], not cfg["summary"], device)
    if companion:
        g = g / 4096.0
        beta = beta / 64.0
    name = cfg["name"] + (" (slow-decay companion)" if companion else "")
    return Problem(name=name, cu_seqlens=cu.to(device), q=q, k=k, v=v,
                   g=g, beta=beta, state=state, l2norm=True, summary=cfg["summary"])


def custom_problem(lengths, hk, hv, dk, dv, seed=0, with_state=False, summary=False,
                   l2norm=True, g_div=1.0, beta_div=1.0, device="cpu") -> Problem:
    """A problem of arbitrary shape with the same distributions."""
    gen = torch.Generator(device=device).manual_seed(seed)
    cu, q, k, v, g, beta, state = _draw(gen, list(lengths), hk, hv, dk, dv, with_state,
                                        not summary, device)
    return Problem(name=f"custom{tuple(lengths)}", cu_seqlens=cu.to(device), q=q, k=k, v=v, g=g / g_div,
                   beta=beta / beta_div, state=state, l2norm=l2norm, summary=summary)


def fused_problem(lengths, hk, hv, dk, dv, seed=0, with_state=False, summary=False, beta_sigmoid=True,
                  safe_gate=True, with_dt_bias=True, a_log_shift=0.0, beta_logit_shift=0.0,
                  device="cpu") -> Problem:
    """Inputs for the gate and beta transforms fused into the kernels.

    q, k, v and the state as in custom_problem.  The raw gate is N(0,1) fp32 and
    the beta logits N(0,1) rounded to bf16 (plus beta_logit_shift).  Per value
    head, a_log = log(A) with A ~ U(1, 16) (plus a_log_shift) and dt_bias the
    inverse softplus of dt, log dt ~ U(log 1e-3, log 1e-1): the shapes of the
    usual Gated DeltaNet layer's initialisation, so that the effective gate
    -exp(a_log) softplus(g + dt_bias) is about -0.1 per token.  Draw order: the
    custom_problem draws, then raw gate, beta logits, A, dt.
    """
    gen = torch.Generator(device=device).manual_seed(seed)
    cu, q, k, v, _, _, state = _draw(gen, list(lengths), hk, hv, dk, dv, with_state, not summary, device)
    T = int(sum(lengths))

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)

    def rand(*shape):
        return torch.rand(*shape, generator=gen, dtype=torch.float32, device=device)

    g_raw = randn(T, hv)
    logits = (randn(T, hv) + beta_logit_shift).to(torch.bfloat16)
    A = 1.0 + 15.0 * rand(hv)
    dt = torch.exp(np.log(1e-3) + (np.log(1e-1) - np.log(1e-3)) * rand(hv))
    a_log = (torch.log(A) + a_log_shift) if safe_gate else None
    dt_bias = (dt + torch.log(-torch.expm1(-dt))) if (safe_gate and with_dt_bias) else None
    if safe_gate:
        g = g_raw
    else:
        g = -torch.nn.functional.softplus(g_raw)
    beta = logits if beta_sigmoid else torch.sigmoid(logits.float())
    return Problem(name=f"fused{tuple(lengths)}", cu_seqlens=cu.to(device), q=q, k=k, v=v, g=g, beta=beta,
                   state=state, l2norm=True, summary=summary, beta_sigmoid=beta_sigmoid, a_log=a_log,
                   dt_bias=dt_bias)


def gdp_problem(lengths, nh, hk, hv, dk, dv, seed=0, with_state=False, summary=False, g_div=1.0,
                beta_div=1.0, device="cpu") -> Problem:
    """Gated Delta Product inputs: q and g one row per token, k, v and beta nh rows
    per token (update-major: the updates of token t are rows t nh .. t nh + nh - 1).
    Distributions as in custom_problem.  Draw order: the custom_problem draws over the
    T nh update rows (q, g and the state drawn that way and q, g cut to the first T
    rows), so nh = 1 gives custom_problem's tensors."""
    T = int(sum(lengths))
    gen = torch.Generator(device=device).manual_seed(seed)
    rows = [L * nh for L in lengths]
    cu_u, q, k, v, g, beta, state = _draw(gen, rows, hk, hv, dk, dv, with_state, not summary, device)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(list(lengths), dtype=torch.int64), 0).to(torch.int32)
    return Problem(name=f"gdp{nh}{tuple(lengths)}", cu_seqlens=cu.to(device),
                   q=None if q is None else q[:T].contiguous(), k=k, v=v, g=(g[:T] / g_div).contiguous(),
                   beta=beta / beta_div, state=state, l2norm=True, summary=summary, num_householder=nh)
