"""GPU parity of the forward's state series (la_gdn_fwd_ex with
checkpoint_every_n_tokens: one entry every n tokens strictly before each
sequence end, entry j the state after j n tokens; the "Linear Attention"
page, "States and checkpoints") against the fp64 oracle's series."""
import numpy as np
import pytest
import torch

import gated_delta_rule_50_amd as la
from oracle import Oracle, rel_l2
from workloads import custom_problem, fused_problem, make_problem

from gpu_helpers import TOL_O, TOL_STATE, assert_o_state, assert_states, f64, gpu_fwd, note

pytestmark = pytest.mark.gpu

TOL_CK_BF16 = 1e-2   # bf16 rows: the row rounding alone is ~2e-3


def fwd_ck(p, every, dtype=torch.float32, **kw):
    g = p.to("cuda")
    out, fin, ck = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                    checkpoint_every_n_tokens=every, checkpoint_dtype=dtype,
                                    beta_sigmoid=p.beta_sigmoid, a_log=g.a_log, dt_bias=g.dt_bias, **kw)
    torch.cuda.synchronize()
    return out, fin, ck


@pytest.mark.parametrize("every", [64, 128])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
def test_series_fp32_against_oracle(every, dk, dv):
    p = custom_problem((1, 63, 64, 65, 0, 200, 257), hk=2, hv=4, dk=dk, dv=dv, seed=71, with_state=True)
    note(f"series fp32 every={every} K={dk} V={dv}")
    out, fin, ck = fwd_ck(p, every)
    ref = Oracle(p).run_all(checkpoint_every=every)
    assert ck.shape[0] == ref["checkpoints"].shape[0] == la.checkpoint_entries(p.cu_seqlens, every)
    assert_states(ck, ref["checkpoints"], TOL_STATE, "state series")
    assert_o_state(out, fin, ref)
    # entry 0 of every non-empty sequence is its initial state, bit for bit
    lens = [1, 63, 64, 65, 0, 200, 257]
    base = 0
    for s, L in enumerate(lens):
        if L:
            assert torch.equal(ck[base].cpu(), p.state[s])
        base += -(-L // every)


def test_series_bf16_rows_and_outputs_unchanged():
    p = custom_problem((100, 257), hk=2, hv=4, dk=128, dv=128, seed=72, with_state=True)
    note("series bf16")
    out, fin, ck = fwd_ck(p, 64, torch.bfloat16)
    assert ck.dtype == torch.bfloat16
    ref = Oracle(p).run_all(checkpoint_every=64)
    assert_states(ck, ref["checkpoints"], TOL_CK_BF16, "state series")
    o0, f0 = gpu_fwd(p)
    assert torch.equal(out, o0) and torch.equal(fin, f0)


def test_series_capacity_limits_writes():
    p = custom_problem((300,), hk=1, hv=2, dk=64, dv=64, seed=73, with_state=True)
    full = la.checkpoint_entries(p.cu_seqlens, 64)          # 5
    buf = torch.full((full - 2, 2, 64, 64), 7.0, device="cuda")
    note("series capacity")
    out, fin, ck = fwd_ck(p, 64, checkpoints=buf)
    ref = Oracle(p).run_all(checkpoint_every=64)["checkpoints"]
    assert_states(ck, ref[:full - 2], TOL_STATE, "state series")


def test_series_varlen_h16_and_fused_transforms():
    p = make_problem(2)
    note("series varlen H=16")
    out, fin, ck = fwd_ck(p, 64)
    ref = Oracle(p).run_all(checkpoint_every=64)
    assert_states(ck, ref["checkpoints"], TOL_STATE, "state series")
    q = fused_problem((300, 129), hk=2, hv=4, dk=128, dv=128, seed=74, with_state=True)
    note("series with fused gate and beta")
    out, fin, ck = fwd_ck(q, 128)
    ref = Oracle(q).run_all(checkpoint_every=128)
    assert_states(ck, ref["checkpoints"], TOL_STATE, "state series")
    assert_o_state(out, None, ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_series_two_tile_workgroups(dtype):
    # 40 sequences x 2 value heads x 4 value tiles = 320 one-tile inter workgroups, more than
    # one per CU and at most two: the forward with the series runs two 32-column tiles per
    # workgroup.  Against the oracle, and sequences alone (one tile per workgroup) bit for bit.
    lens = [(i * 53) % 300 + 1 for i in range(40)]
    p = custom_problem(lens, hk=1, hv=2, dk=128, dv=128, seed=74, with_state=True)
    note(f"series two-tile workgroups {dtype}")
    out, fin, ck = fwd_ck(p, 64, dtype)
    ref = Oracle(p).run_all(checkpoint_every=64)
    assert_states(ck, ref["checkpoints"], TOL_STATE if dtype == torch.float32 else TOL_CK_BF16, "state series")
    assert_o_state(out, fin, ref)
    cu = p.cu_seqlens.tolist()
    base = [0]
    for L in lens:
        base.append(base[-1] + -(-L // 64))
    for n in [0, 9, 39]:
        sl = slice(cu[n], cu[n + 1])
        alone = type(p)("alone", torch.tensor([0, lens[n]], dtype=torch.int32), p.q[sl].contiguous(),
                        p.k[sl].contiguous(), p.v[sl].contiguous(), p.g[sl].contiguous(), p.beta[sl].contiguous(),
                        p.state[n:n + 1].clone())
        oa, fa, ca = fwd_ck(alone, 64, dtype)
        assert torch.equal(oa, out[sl]) and torch.equal(fa[0], fin[n]), n
        assert torch.equal(ca, ck[base[n]:base[n + 1]]), n
