"""Shared helpers of the GPU tests: run the HIP path on a workloads.Problem
through the C ABI, and compare with the fp64 oracle."""
import dataclasses
import sys

import numpy as np
import torch

import gated_delta_rule_50_amd as la
from oracle import Oracle, rel_l2

TOL_O = 1e-2       # bf16 output, rel-L2
TOL_STATE = 5e-3   # fp32 final / end state and transition, rel-L2


def note(msg: str):
    """Names the case on stdout before a GPU step (flushed)."""
    print(f"[gpu-case] {msg}", flush=True)


def gpu_fwd(p, dev="cuda", initial_state=True, scale=None, **kw):
    g = p.to(dev)
    s0 = g.state if initial_state else None
    out, fin = la.la_gdn_fwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=s0,
                             l2norm=p.l2norm, scale=scale, **kw)
    torch.cuda.synchronize()
    return out, fin


def gpu_summary(p, dev="cuda", start_state=True, **kw):
    g = p.to(dev)
    s0 = g.state if start_state else None
    end, tr = la.la_gdn_summary(g.k, g.v, g.g, g.beta, g.cu_seqlens, start_state=s0,
                                l2norm=p.l2norm, **kw)
    torch.cuda.synchronize()
    return end, tr


def f64(t):
    return t.detach().float().cpu().double().numpy()


# Row by row (one token-head of o, one (sequence, head) state): the whole-tensor bounds
# above can hide a few wrong rows of a large tensor, so every row must also be within
# ROW_FACTOR times its tolerance of its own norm, plus a floor of that tolerance times the
# tensor's rms row norm (rows near zero).
ROW_FACTOR = 5.0


def assert_rows_close(x, ref, tol, what):
    """x, ref: [rows..., n] arrays; each last-axis row within ROW_FACTOR * tol."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    if ref.shape[0] == 0:
        return
    err = np.linalg.norm(x - ref, axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    rms = float(np.sqrt(np.mean(nrm ** 2)))
    bound = ROW_FACTOR * tol * (nrm + rms)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows beyond {ROW_FACTOR} x {tol} (first {bad[:5].tolist()}, "
                           f"worst err/norm {float(np.max(err / np.maximum(nrm, 1e-30))):.3e})")


def assert_o_state(out, fin, ref, tol_o=TOL_O, tol_s=TOL_STATE):
    """o and final states against the oracle's: whole-tensor rel-L2 and row by row
    (fin may be None when only o is compared)."""
    eo = rel_l2(f64(out), ref["o"])
    assert eo <= tol_o, f"o rel-L2 {eo:.3e} > {tol_o}"
    assert_rows_close(f64(out), ref["o"], tol_o, "o rows")
    if fin is not None:
        es = rel_l2(f64(fin), ref["state"])
        assert es <= tol_s, f"final state rel-L2 {es:.3e} > {tol_s}"
        K, V = ref["state"].shape[-2:]
        assert_rows_close(f64(fin).reshape(-1, K * V), ref["state"].reshape(-1, K * V), tol_s, "final states")


def assert_states(x, ref, tol, what):
    """[..., K, V] fp32 states (final states, series entries) against the oracle's:
    whole-tensor rel-L2 and one K x V state per row."""
    ref = np.asarray(ref)
    K, V = ref.shape[-2:]
    e = rel_l2(f64(x), ref)
    assert e <= tol, f"{what}: rel-L2 {e:.3e} > {tol}"
    assert_rows_close(f64(x).reshape(-1, K * V), ref.reshape(-1, K * V), tol, what)


def assert_summary(end, tr, ref, tol=TOL_STATE, check_transition=True):
    """End states and transitions against the oracle's: whole-tensor rel-L2 and row by
    row (one (sequence, head) state or transition per row)."""
    K, V = ref["state"].shape[-2:]
    ee = rel_l2(f64(end), ref["state"])
    assert ee <= tol, f"end state rel-L2 {ee:.3e} > {tol}"
    assert_rows_close(f64(end).reshape(-1, K * V), ref["state"].reshape(-1, K * V), tol, "end states")
    if check_transition:
        et = rel_l2(f64(tr), ref["transition"])
        assert et <= tol, f"transition rel-L2 {et:.3e} > {tol}"
        assert_rows_close(f64(tr).reshape(-1, K * K), ref["transition"].reshape(-1, K * K), tol, "transitions")


class UnitTally:
    """Whole-tensor rel-L2 and row bounds accumulated unit by unit, for tensors too
    large to assemble in fp64 twice (every unit of the long-context and span
    workloads)."""

    def __init__(self, tol, what):
        self.tol, self.what = tol, what
        self.num = self.den = 0.0
        self.err, self.nrm, self.tag = [], [], []

    def add(self, x, ref, tag, per_unit=True):
        x = np.asarray(x, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
        ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
        d = np.linalg.norm(x - ref, axis=1)
        n = np.linalg.norm(ref, axis=1)
        self.num += float(np.sum(d * d))
        self.den += float(np.sum(n * n))
        self.err.append(d)
        self.nrm.append(n)
        self.tag.append(tag)
        if per_unit and n.size:
            e = float(np.sqrt(np.sum(d * d)) / max(np.sqrt(np.sum(n * n)), 1e-300))
            assert e <= self.tol, f"{self.what} of unit {tag}: rel-L2 {e:.3e} > {self.tol}"

    def check(self):
        e = float(np.sqrt(self.num) / max(np.sqrt(self.den), 1e-300))
        assert e <= self.tol, f"{self.what}: rel-L2 {e:.3e} > {self.tol}"
        err, nrm = np.concatenate(self.err), np.concatenate(self.nrm)
        rms = float(np.sqrt(np.mean(nrm ** 2))) if nrm.size else 0.0
        bad = np.nonzero(~(err <= ROW_FACTOR * self.tol * (nrm + rms)))[0]
        assert bad.size == 0, f"{self.what}: {bad.size} rows beyond {ROW_FACTOR} x {self.tol}"
        return e


def check_fwd_full(p, tol_o=TOL_O, tol_s=TOL_STATE, initial_state=True):
    """Whole-tensor rel-L2 of o and final state against the oracle, and row by row."""
    note(f"fwd full: {p.name} T={p.total_tokens} N={p.num_seqs}")
    out, fin = gpu_fwd(p, initial_state=initial_state)
    ref = Oracle(p, use_initial_state=initial_state).run_all()
    eo = rel_l2(f64(out), ref["o"])
    es = rel_l2(f64(fin), ref["state"])
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= tol_o, f"o rel-L2 {eo:.3e} > {tol_o}"
    assert es <= tol_s, f"final state rel-L2 {es:.3e} > {tol_s}"
    assert_rows_close(f64(out), ref["o"], tol_o, "o rows")
    K, V = ref["state"].shape[-2:]
    assert_rows_close(f64(fin).reshape(-1, K * V), ref["state"].reshape(-1, K * V), tol_s, "final states")
    return out, fin, ref, eo, es
