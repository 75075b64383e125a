"""A seeded sweep of random shapes and options against the fp64 oracle: the forward (plain,
with the fused gate and beta transforms, or with the state series), the span summary, the
full backward, the summary's state-gradient mirror and the Gated Delta Product (forward and
summary, 2 to 4 updates per token).  Each case draws its own sequence
lengths (empty, single-token, partial-chunk, whole-chunk and multi-chunk sequences),
head counts (grouped or not), head dims and initial state from a generator seeded by the
case number, so that the kernel variants (one or two tiles per inter workgroup, grouped
and ungrouped backward) meet combinations the targeted tests do not name.  Tolerances as
in the targeted tests; every forward case also runs one of its sequences alone and
compares o and the final state bit for bit (the "Linear Attention" page, "Semantics worth
knowing", batch_invariant)."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_50_amd as la
import oracle
from oracle import Oracle, rel_l2
from workloads import custom_problem, fused_problem, gdp_problem

from gpu_helpers import TOL_STATE, assert_o_state, assert_rows_close, assert_states, assert_summary, f64, note

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-2


def _lengths(rng, n):
    out = []
    for _ in range(n):
        kind = rng.random()
        if kind < 0.08:
            out.append(0)
        elif kind < 0.35:
            out.append(int(rng.integers(1, 65)))
        elif kind < 0.5:
            out.append(64 * int(rng.integers(1, 6)))
        else:
            out.append(int(rng.integers(65, 420)))
    if not any(out):
        out[0] = int(rng.integers(1, 300))
    return tuple(out)


def _heads(rng, max_hv):
    while True:
        hk = int(rng.choice([1, 2, 4]))
        hv = hk * int(rng.choice([1, 2, 4]))
        if hv <= max_hv:
            return hk, hv


def _dims(rng):
    return int(rng.choice([64, 128])), int(rng.choice([64, 128]))


def _alone(p, s):
    """Sequence s of p as a problem of its own (same tensors, sliced)."""
    cu = p.cu_seqlens.tolist()
    a, b = cu[s], cu[s + 1]
    sl = slice(a, b)
    return dataclasses.replace(
        p, cu_seqlens=torch.tensor([0, b - a], dtype=torch.int32), q=p.q[sl].contiguous(),
        k=p.k[sl].contiguous(), v=p.v[sl].contiguous(), g=p.g[sl].contiguous(), beta=p.beta[sl].contiguous(),
        state=None if p.state is None else p.state[s:s + 1].contiguous())


def _fwd(p, every=0):
    g = p.to("cuda")
    out, fin, ck = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                    beta_sigmoid=p.beta_sigmoid, a_log=g.a_log, dt_bias=g.dt_bias,
                                    checkpoint_every_n_tokens=every, checkpoint_dtype=torch.float32)
    torch.cuda.synchronize()
    return out, fin, ck


@pytest.mark.parametrize("case", range(24))
def test_random_forward(case):
    rng = np.random.default_rng(5000 + case)
    n = int(rng.integers(1, 13))
    lens = _lengths(rng, n)
    hk, hv = _heads(rng, 16)
    dk, dv = _dims(rng)
    with_state = bool(rng.random() < 0.6)
    mode = ("plain", "fused", "series")[case % 3]
    if mode == "fused":
        p = fused_problem(lens, hk=hk, hv=hv, dk=dk, dv=dv, seed=5100 + case, with_state=with_state)
    else:
        p = custom_problem(lens, hk=hk, hv=hv, dk=dk, dv=dv, seed=5100 + case, with_state=with_state)
    every = int(rng.choice([64, 128])) if mode == "series" else 0
    note(f"random fwd {case}: {mode} lens={lens} HK={hk} HV={hv} K={dk} V={dv} state={with_state} every={every}")
    out, fin, ck = _fwd(p, every)
    ref = Oracle(p).run_all(checkpoint_every=every)
    assert_o_state(out, fin, ref)
    if every:
        assert ck.shape[0] == ref["checkpoints"].shape[0]
        assert_states(ck, ref["checkpoints"], TOL_STATE, "state series")
    # batch invariance: the longest sequence run alone gives the same bits
    s = int(np.argmax(lens))
    a = _alone(p, s)
    out1, fin1, _ = _fwd(a, every)
    cu = p.cu_seqlens.tolist()
    assert torch.equal(out[cu[s]:cu[s + 1]].cpu(), out1.cpu()), "o of the sequence run alone differs"
    assert torch.equal(fin[s].cpu(), fin1[0].cpu()), "final state of the sequence run alone differs"


@pytest.mark.parametrize("case", range(8))
def test_random_summary(case):
    rng = np.random.default_rng(6000 + case)
    lens = _lengths(rng, int(rng.integers(1, 13)))
    hk, hv = _heads(rng, 16)
    dk, dv = _dims(rng)
    # slow decay, so that the transitions stay well away from zero
    p = custom_problem(lens, hk=hk, hv=hv, dk=dk, dv=dv, seed=6100 + case, with_state=bool(rng.random() < 0.6),
                       summary=True, g_div=4096.0, beta_div=64.0)
    note(f"random summary {case}: lens={lens} HK={hk} HV={hv} K={dk} V={dv}")
    g = p.to("cuda")
    end, tr = la.la_gdn_summary(g.k, g.v, g.g, g.beta, g.cu_seqlens, start_state=g.state, l2norm=p.l2norm)
    torch.cuda.synchronize()
    ref = Oracle(p).run_all(want_o=False, want_transition=True)
    assert_summary(end, tr, ref)


def _grads_close(got, ref, names, tol):
    for name in names:
        x, r = f64(got[name]), ref[name]
        e = rel_l2(x, r)
        assert np.isfinite(e) and e <= tol, f"{name}: rel-L2 {e:.3e} > {tol}"
        if r.ndim >= 2 and r.size:
            last = r.shape[-1] * (r.shape[-2] if name == "d_init" else 1)
            assert_rows_close(x.reshape(-1, last), r.reshape(-1, last), tol, f"{name} rows")


@pytest.mark.parametrize("case", range(8))
def test_random_backward(case):
    rng = np.random.default_rng(7000 + case)
    lens = _lengths(rng, int(rng.integers(1, 13)))
    hk, hv = _heads(rng, 16)
    dk, dv = _dims(rng)
    with_state = bool(rng.random() < 0.6)
    p = custom_problem(lens, hk=hk, hv=hv, dk=dk, dv=dv, seed=7100 + case, with_state=with_state)
    note(f"random bwd {case}: lens={lens} HK={hk} HV={hv} K={dk} V={dv} state={with_state}")
    gen = torch.Generator().manual_seed(7200 + case)
    T = p.total_tokens
    d_out = torch.randn((T, hv, dv), generator=gen).to(torch.bfloat16)
    d_fin = torch.randn((p.num_seqs, hv, dk, dv), generator=gen)
    g = p.to("cuda")
    got = la.la_gdn_bwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, d_out.cuda(), initial_state=g.state,
                        d_final_state=d_fin.cuda(), l2norm=p.l2norm)
    torch.cuda.synchronize()
    got["d_init"] = got.pop("d_initial_state")
    ref = oracle.backward(p, d_o=d_out.double().numpy(), d_final=d_fin.double().numpy())
    _grads_close(got, ref, ("dq", "dk", "dv", "dg", "dbeta", "d_init"), TOL_BWD)


@pytest.mark.parametrize("case", range(4))
def test_random_summary_bwd(case):
    rng = np.random.default_rng(8000 + case)
    lens = _lengths(rng, int(rng.integers(1, 9)))
    hk, hv = _heads(rng, 8)
    dk, dv = _dims(rng)
    p = custom_problem(lens, hk=hk, hv=hv, dk=dk, dv=dv, seed=8100 + case)
    p = dataclasses.replace(p, g=p.g / 8.0, beta=p.beta / 2.0)
    note(f"random summary bwd {case}: lens={lens} HK={hk} HV={hv} K={dk} V={dv}")
    gen = torch.Generator().manual_seed(8200 + case)
    d_out = torch.randn((p.total_tokens, hv, dv), generator=gen).to(torch.bfloat16)
    d_end = torch.randn((p.num_seqs, hv, dk, dv), generator=gen)
    g = p.to("cuda")
    got = la.la_gdn_summary_bwd(g.q, g.k, g.g, g.beta, g.cu_seqlens, d_out.cuda(), d_end.cuda(), l2norm=p.l2norm)
    torch.cuda.synchronize()
    ref = oracle.backward(p, d_o=d_out.double().numpy(), d_final=d_end.double().numpy())["d_init"]
    _grads_close({"d_init": got}, {"d_init": ref}, ("d_init",), TOL_STATE)


@pytest.mark.parametrize("case", range(8))
def test_random_gated_delta_product(case):
    rng = np.random.default_rng(9000 + case)
    lens = _lengths(rng, int(rng.integers(1, 9)))
    nh = int(rng.choice([2, 3, 4]))
    hk, hv = _heads(rng, 8)
    dk, dv = _dims(rng)
    with_state = bool(rng.random() < 0.6)
    summary = case % 4 == 3
    # the summary on slow decay, so that its transitions stay well away from zero
    p = gdp_problem(lens, nh, hk=hk, hv=hv, dk=dk, dv=dv, seed=9100 + case, with_state=with_state,
                    summary=summary, g_div=4096.0 if summary else 1.0, beta_div=64.0 if summary else 1.0)
    note(f"random gdp {case}: n={nh} summary={summary} lens={lens} HK={hk} HV={hv} K={dk} V={dv} state={with_state}")
    g = p.to("cuda")
    if summary:
        end, tr = la.la_gdn_summary_ex(g.k, g.v, g.g, g.beta, g.cu_seqlens, start_state=g.state,
                                       num_householder=nh)
        torch.cuda.synchronize()
        assert_summary(end, tr, Oracle(p).run_all(want_o=False, want_transition=True))
    else:
        out, fin, _ = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                       num_householder=nh)
        torch.cuda.synchronize()
        assert_o_state(out, fin, Oracle(p).run_all())
