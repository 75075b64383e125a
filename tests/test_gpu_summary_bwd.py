"""GPU parity of the span summary's mirror for the state gradient (la_gdn_summary_bwd)
against the fp64 oracle's backward (its gradient of the initial state for the same output
and end-state gradients), and its invariants."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_50_amd as la
import oracle
from oracle import rel_l2
from workloads import custom_problem

from gpu_helpers import TOL_STATE, assert_rows_close, f64, note

pytestmark = pytest.mark.gpu


def _inputs(p, seed):
    gen = torch.Generator().manual_seed(seed)
    T, HV, V = p.v.shape
    K = p.k.shape[2]
    d_out = torch.randn((T, HV, V), generator=gen).to(torch.bfloat16)
    d_end = torch.randn((p.num_seqs, HV, K, V), generator=gen)
    return d_out, d_end


def _check(p, seed, scale=None):
    d_out, d_end = _inputs(p, seed)
    g = p.to("cuda")
    note(f"summary bwd: {p.name} l2norm={p.l2norm}")
    got = la.la_gdn_summary_bwd(g.q, g.k, g.g, g.beta, g.cu_seqlens, d_out.cuda(), d_end.cuda(),
                                l2norm=p.l2norm, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.backward(p, d_o=d_out.double().numpy(), d_final=d_end.double().numpy(), scale=scale)["d_init"]
    assert rel_l2(f64(got), ref) <= TOL_STATE, rel_l2(f64(got), ref)
    K, V = ref.shape[-2:]
    assert_rows_close(f64(got).reshape(-1, K * V), ref.reshape(-1, K * V), TOL_STATE, "d_start rows")
    return got, d_end


def _problem(lengths, dk, dv, seed, l2norm=True):
    p = custom_problem(lengths, hk=2, hv=4, dk=dk, dv=dv, seed=seed, l2norm=l2norm)
    return dataclasses.replace(p, g=p.g / 8.0, beta=p.beta / 2.0)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_summary_bwd_matches_oracle(dk, dv):
    got, d_end = _check(_problem((1, 63, 64, 65, 200, 0), dk, dv, seed=121), seed=122)
    # the empty sequence passes its end-state gradient through unchanged
    assert torch.equal(got[5].cpu(), d_end[5])


def test_summary_bwd_no_l2norm_custom_scale():
    p = _problem((30, 90), 128, 128, seed=123, l2norm=False)
    p = dataclasses.replace(p, q=(p.q.float() * 0.1).to(torch.bfloat16), k=(p.k.float() * 0.1).to(torch.bfloat16))
    _check(p, seed=124, scale=0.3)


def test_summary_bwd_long_span():
    _check(_problem((2000,), 128, 128, seed=125), seed=126)


def test_summary_bwd_null_end_gradient_is_zeros_bitwise():
    p = _problem((50, 70), 128, 128, seed=127)
    d_out, d_end = _inputs(p, 128)
    g = p.to("cuda")
    note("summary bwd: NULL d_end against zeros")
    a = la.la_gdn_summary_bwd(g.q, g.k, g.g, g.beta, g.cu_seqlens, d_out.cuda(), None)
    b = la.la_gdn_summary_bwd(g.q, g.k, g.g, g.beta, g.cu_seqlens, d_out.cuda(), torch.zeros_like(d_end).cuda())
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_summary_bwd_bad_cu_seqlens_writes_nothing():
    p = _problem((10, 20), 64, 64, seed=129)
    d_out, d_end = _inputs(p, 130)
    g = p.to("cuda")
    desc = la.make_desc(g.k, g.v, g.g, g.beta, 2, q=g.q)
    ws = la.alloc_workspace(desc, True, "cuda")
    for bad in ([0, 25, 20], [1, 10, 30], [0, 10, 31]):
        note(f"summary bwd: bad cu_seqlens {bad}")
        out = torch.full((2, 4, 64, 64), 3.0, device="cuda")
        la.la_gdn_summary_bwd(g.q, g.k, g.g, g.beta, torch.tensor(bad, dtype=torch.int32, device="cuda"),
                              d_out.cuda(), d_end.cuda(), d_start_state=out, workspace=ws)
        assert la.la_gdn_device_status(ws) == la.LA_DEVICE_BAD_CU_SEQLENS
        assert bool((out == 3.0).all())
    la.la_gdn_summary_bwd(g.q, g.k, g.g, g.beta, g.cu_seqlens, d_out.cuda(), d_end.cuda(), workspace=ws)
    assert la.la_gdn_device_status(ws) == la.LA_DEVICE_OK


def test_summary_bwd_strided_views_equal_contiguous_bitwise():
    """q, k and d_out as column slices of wider per-token buffers (the strides of the
    descriptor), against contiguous copies: the same bits."""
    p = _problem((40, 0, 150), 64, 128, seed=131)
    d_out, d_end = _inputs(p, 132)
    g = p.to("cuda")
    T, HK, K = p.k.shape
    HV, V = d_out.shape[1], d_out.shape[2]
    wide = torch.zeros((T, 2 * HK * K + 16), dtype=torch.bfloat16, device="cuda")
    wide[:, :HK * K] = g.q.reshape(T, HK * K)
    wide[:, HK * K + 8:2 * HK * K + 8] = g.k.reshape(T, HK * K)
    q_v = wide[:, :HK * K].view(T, HK, K)
    k_v = wide[:, HK * K + 8:2 * HK * K + 8].view(T, HK, K)
    dwide = torch.zeros((T, HV, V + 8), dtype=torch.bfloat16, device="cuda")
    dwide[:, :, :V] = d_out.cuda()
    d_v = dwide[:, :, :V]
    note("summary bwd: strided q, k, d_out")
    a = la.la_gdn_summary_bwd(g.q, g.k, g.g, g.beta, g.cu_seqlens, d_out.cuda(), d_end.cuda())
    b = la.la_gdn_summary_bwd(q_v, k_v, g.g, g.beta, g.cu_seqlens, d_v, d_end.cuda())
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_summary_bwd_slow_decay_every_chunk_matters():
    # gate / 4096 and beta / 64: the start-state gradient depends on every chunk of the span
    # (under the faster gates above only the first chunks reach it)
    p = custom_problem((2000, 300), hk=2, hv=4, dk=128, dv=128, seed=133, g_div=4096.0, beta_div=64.0)
    _check(p, seed=134)


def test_summary_bwd_two_tile_workgroups():
    # 5 spans x 16 heads x 4 value tiles = 320 one-tile workgroups, more than one per CU and at
    # most two: the reverse pass runs with two 32-column tiles per workgroup (slow decay, so
    # that every chunk reaches the start-state gradient)
    p = custom_problem((130, 64, 1, 300, 77), hk=4, hv=16, dk=128, dv=128, seed=135, g_div=4096.0,
                       beta_div=64.0)
    _check(p, seed=136)
