"""GPU parity of the Gated Delta Product (la_gdn_fwd_ex / la_gdn_summary_ex with
num_householder = n: k, v and beta n update rows per token, update-major or token-major; q, g
and o one row per token) against the fp64 oracle's token recurrence with n
updates per token.  Tolerances as for GDN."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_50_amd as la
from oracle import Oracle, rel_l2
from workloads import gdp_problem

from gpu_helpers import TOL_O, TOL_STATE, assert_o_state, assert_summary, f64, gpu_fwd, note

pytestmark = pytest.mark.gpu


def gdp_fwd(p):
    g = p.to("cuda")
    out, fin, _ = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                   num_householder=p.num_householder)
    torch.cuda.synchronize()
    return out, fin


def check(p):
    note(f"gdp fwd: {p.name} n={p.num_householder}")
    out, fin = gdp_fwd(p)
    ref = Oracle(p).run_all()
    assert_o_state(out, fin, ref)
    return out, fin


@pytest.mark.parametrize("nh", [2, 3])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128)])
def test_gdp_ragged(nh, dk, dv):
    # lengths in tokens: chunks of 64 update rows then start inside a token for n = 3
    check(gdp_problem((1, 21, 32, 33, 100, 150), nh, hk=2, hv=4, dk=dk, dv=dv, seed=91, with_state=True))


def test_gdp_larger():
    check(gdp_problem((700, 1300), 2, hk=4, hv=8, dk=128, dv=128, seed=92, with_state=True))


def test_gdp_one_update_is_the_plain_call_bitwise():
    p = gdp_problem((100, 257), 1, hk=2, hv=4, dk=128, dv=128, seed=93, with_state=True)
    note("gdp n=1 vs plain")
    o1, f1 = gdp_fwd(p)
    o2, f2 = gpu_fwd(p)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_gdp_summary_slow_decay():
    p = gdp_problem((1, 40, 100, 150), 2, hk=2, hv=2, dk=128, dv=128, seed=94, with_state=True, summary=True,
                    g_div=4096.0, beta_div=64.0)
    g = p.to("cuda")
    note("gdp summary n=2")
    end, tr = la.la_gdn_summary_ex(g.k, g.v, g.g, g.beta, g.cu_seqlens, start_state=g.state, num_householder=2)
    torch.cuda.synchronize()
    ref = Oracle(p).run_all(want_o=False, want_transition=True)
    assert_summary(end, tr, ref)
    assert np.abs(ref["transition"]).max() > 0.05


def test_gdp_with_fused_gate_and_beta():
    # raw gate per token, bf16 beta logits per update row, safe-gate parameters per value head
    p = gdp_problem((1, 30, 50, 130), 2, hk=2, hv=4, dk=128, dv=128, seed=95, with_state=True)
    gen = torch.Generator().manual_seed(96)
    g_raw = torch.randn(p.g.shape, generator=gen)
    logits = torch.randn(p.beta.shape, generator=gen).to(torch.bfloat16)
    a_log = torch.log(1.0 + 15.0 * torch.rand(4, generator=gen))
    dt = torch.exp(np.log(1e-3) + (np.log(1e-1) - np.log(1e-3)) * torch.rand(4, generator=gen))
    dt_bias = dt + torch.log(-torch.expm1(-dt))
    p = dataclasses.replace(p, g=g_raw, beta=logits, beta_sigmoid=True, a_log=a_log, dt_bias=dt_bias)
    g = p.to("cuda")
    note("gdp n=2 with fused gate and beta")
    out, fin, _ = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                   num_householder=2, beta_sigmoid=True, a_log=g.a_log, dt_bias=g.dt_bias)
    torch.cuda.synchronize()
    ref = Oracle(p).run_all()
    assert_o_state(out, fin, ref)


def token_major(p, pad=8):
    """k, v and beta of an update-major problem on the GPU as token-major views into joint
    per-token buffers ([T, n HV V | n HK K | pad] for v and k, [T, n HV | pad] for beta), the
    layout of per-token column slices of one projection: neither token stride is n times
    its update stride."""
    T, n = p.total_tokens, p.num_householder
    HK, K, HV, V = p.k.shape[1], p.k.shape[2], p.v.shape[1], p.v.shape[2]
    wv, wk = n * HV * V, n * HK * K
    joint = torch.zeros(T, wv + wk + pad, dtype=torch.bfloat16, device="cuda")
    joint[:, :wv] = p.v.reshape(T, wv).cuda()
    joint[:, wv:wv + wk] = p.k.reshape(T, wk).cuda()
    bj = torch.zeros(T, n * HV + pad // 2, dtype=p.beta.dtype, device="cuda")
    bj[:, :n * HV] = p.beta.reshape(T, n * HV).cuda()
    return (joint[:, wv:wv + wk].view(T, n, HK, K), joint[:, :wv].view(T, n, HV, V),
            bj[:, :n * HV].view(T, n, HV))


@pytest.mark.parametrize("nh", [2, 3])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 128)])
def test_gdp_token_major_forward(nh, dk, dv):
    """Token-major k, v and beta (the pages' second GDP layout) give the update-major
    call's results bit for bit, and so the oracle's."""
    p = gdp_problem((1, 21, 33, 100, 150), nh, hk=2, hv=4, dk=dk, dv=dv, seed=97, with_state=True)
    out_u, fin_u = check(p)
    g = p.to("cuda")
    k, v, beta = token_major(p)
    assert k.stride(0) != nh * k.stride(1)
    note(f"gdp token-major fwd n={nh} dk={dk} dv={dv}")
    out, fin, _ = la.la_gdn_fwd_ex(g.q, k, v, g.g, beta, g.cu_seqlens, initial_state=g.state, num_householder=nh)
    torch.cuda.synchronize()
    assert torch.equal(out, out_u) and torch.equal(fin, fin_u)


def test_gdp_token_major_summary_and_fused_beta():
    """The summary from token-major operands, and the forward with token-major bf16 beta
    logits, against their update-major calls bit for bit."""
    p = gdp_problem((1, 40, 100, 150), 3, hk=2, hv=2, dk=128, dv=128, seed=98, with_state=True, summary=True,
                    g_div=4096.0, beta_div=64.0)
    g = p.to("cuda")
    k, v, beta = token_major(p)
    note("gdp token-major summary n=3")
    end_u, tr_u = la.la_gdn_summary_ex(g.k, g.v, g.g, g.beta, g.cu_seqlens, start_state=g.state, num_householder=3)
    end, tr = la.la_gdn_summary_ex(k, v, g.g, beta, g.cu_seqlens, start_state=g.state, num_householder=3)
    torch.cuda.synchronize()
    ref = Oracle(p).run_all(want_o=False, want_transition=True)
    assert_summary(end_u, tr_u, ref)
    assert torch.equal(end, end_u) and torch.equal(tr, tr_u)

    q = gdp_problem((1, 30, 130), 2, hk=2, hv=4, dk=128, dv=128, seed=99, with_state=True)
    logits = torch.randn(q.beta.shape, generator=torch.Generator().manual_seed(100)).to(torch.bfloat16)
    q = dataclasses.replace(q, beta=logits, beta_sigmoid=True)
    gq = q.to("cuda")
    k, v, beta = token_major(q)
    note("gdp token-major fwd n=2 with bf16 beta logits")
    o_u, f_u, _ = la.la_gdn_fwd_ex(gq.q, gq.k, gq.v, gq.g, gq.beta, gq.cu_seqlens, initial_state=gq.state,
                                   beta_sigmoid=True, num_householder=2)
    o_t, f_t, _ = la.la_gdn_fwd_ex(gq.q, k, v, gq.g, beta, gq.cu_seqlens, initial_state=gq.state,
                                   beta_sigmoid=True, num_householder=2)
    torch.cuda.synchronize()
    ref = Oracle(q).run_all()
    assert_o_state(o_u, f_u, ref)
    assert torch.equal(o_t, o_u) and torch.equal(f_t, f_u)


@pytest.mark.parametrize("nh", [5, 63, 64])
def test_gdp_token_major_many_updates(nh):
    """Chunks that start at every phase of a token (n = 5, 63) or always at a token's
    first update (n = 64): token-major equal to update-major bit for bit, both against
    the oracle."""
    p = gdp_problem((1, 2, 7, 13), nh, hk=1, hv=2, dk=64, dv=128, seed=101, with_state=True, g_div=8.0,
                    beta_div=4.0)
    out_u, fin_u = check(p)
    g = p.to("cuda")
    k, v, beta = token_major(p)
    note(f"gdp token-major fwd n={nh}")
    out, fin, _ = la.la_gdn_fwd_ex(g.q, k, v, g.g, beta, g.cu_seqlens, initial_state=g.state, num_householder=nh)
    torch.cuda.synchronize()
    assert torch.equal(out, out_u) and torch.equal(fin, fin_u)
