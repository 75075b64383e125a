"""GPU parity of the full backward (la_gdn_bwd) against the fp64 oracle's backward, which is
pinned by torch autograd and central differences (test_oracle_pins.py).

Tolerance: rel-L2 <= 1e-2 for every gradient (dq, dk, dv, dg, dbeta, d_initial_state), over
the whole tensor and, within five times that, row by row.  The chunked fp64 model with the
kernels' bf16 rounding points (chunked_model.py) predicts about 2.5e-3 on these inputs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_50_amd as la
import oracle
from oracle import rel_l2
from workloads import Problem, custom_problem, make_problem

from gpu_helpers import assert_rows_close, f64, note

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-2
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_init")


def upstream(p, seed, with_final=True):
    gen = torch.Generator().manual_seed(seed)
    T, HV, V = p.v.shape
    K = p.k.shape[2]
    d_out = torch.randn((T, HV, V), generator=gen).to(torch.bfloat16)
    d_fin = torch.randn((p.num_seqs, HV, K, V), generator=gen) if with_final else None
    return d_out, d_fin


def gpu_bwd(p, d_out, d_fin, scale=None, initial_state=True):
    g = p.to("cuda")
    res = la.la_gdn_bwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, d_out.cuda(),
                        initial_state=g.state if initial_state else None,
                        d_final_state=None if d_fin is None else d_fin.cuda(), l2norm=p.l2norm, scale=scale)
    torch.cuda.synchronize()
    res["d_init"] = res.pop("d_initial_state")
    return res


def check_bwd(p, seed, scale=None, with_final=True, tol=TOL_BWD):
    note(f"bwd: {p.name} T={p.total_tokens} N={p.num_seqs} HK={p.num_qk_heads} HV={p.num_v_heads} "
         f"K={p.head_dim_k} V={p.head_dim_v} l2norm={p.l2norm}")
    d_out, d_fin = upstream(p, seed, with_final)
    got = gpu_bwd(p, d_out, d_fin, scale=scale)
    pp = p if p.state is not None else dataclasses.replace(p, state=None)
    ref = oracle.backward(pp, d_o=d_out.double().numpy(), d_final=None if d_fin is None else d_fin.double().numpy(),
                          scale=scale)
    errs = {}
    for name in NAMES:
        x, r = f64(got[name]), ref[name]
        e = rel_l2(x, r)
        errs[name] = e
        assert np.isfinite(e) and e <= tol, f"{name}: rel-L2 {e:.3e} > {tol}"
        if r.ndim >= 2 and r.size:
            last = r.shape[-1] if name not in ("d_init",) else r.shape[-1] * r.shape[-2]
            assert_rows_close(x.reshape(-1, last), r.reshape(-1, last), tol, f"{name} rows")
    print("bwd rel-L2: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    return got, ref


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_backward_ragged_all_head_dims(dk, dv):
    # ragged lengths with a length-1, an exact-chunk and a partial-chunk sequence, grouped
    # heads (2 q/k heads, 4 value heads) and an initial state
    check_bwd(custom_problem((1, 63, 64, 65, 130, 200), hk=2, hv=4, dk=dk, dv=dv, seed=201, with_state=True), 202)


def test_backward_slow_decay_every_chunk_matters():
    # gate / 4096 and beta / 64: the state and its gradient reach across all 12 chunks
    p = custom_problem((700, 64), hk=1, hv=4, dk=128, dv=128, seed=203, with_state=True, g_div=4096.0,
                       beta_div=64.0)
    got, ref = check_bwd(p, 204)
    # not vacuous: the initial state's gradient of the first sequence differs from the end
    # gradient it would be with the tokens' contributions dropped
    assert np.linalg.norm(ref["d_init"][0]) > 0.5


def test_backward_varlen_workload():
    # the varlen workload's shapes: T = 4096 (1000 / 1500 / 1596), H = 16, K = V = 128
    check_bwd(make_problem(2), 205)


@pytest.mark.parametrize("hk,hv", [(1, 2), (2, 2)])
def test_backward_no_l2norm_custom_scale_no_final_gradient(hk, hv):
    # hk = hv: one value head per q/k head, where the intra pass applies the q/k chain itself
    p = custom_problem((70, 130), hk=hk, hv=hv, dk=64, dv=64, seed=206, l2norm=False, with_state=True)
    p = dataclasses.replace(p, k=(p.k.float() / 8).to(torch.bfloat16), q=(p.q.float() / 8).to(torch.bfloat16))
    check_bwd(p, 207, scale=0.3, with_final=False)


def test_backward_zero_initial_state_and_empty_sequences():
    p = custom_problem((0, 5, 0, 129, 0), hk=2, hv=2, dk=128, dv=128, seed=208)
    got, ref = check_bwd(p, 209)
    d_out, d_fin = upstream(p, 209)
    # an empty sequence passes the final-state gradient through to the initial state
    for n in (0, 2, 4):
        assert torch.equal(got["d_init"][n].cpu(), d_fin[n])


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_backward_one_value_head_per_qk_head(dk, dv):
    # G = 1 with ragged lengths and an initial state: dq and dk come straight from the intra pass
    check_bwd(custom_problem((1, 63, 64, 65, 130, 200), hk=3, hv=3, dk=dk, dv=dv, seed=217, with_state=True), 218)


def test_backward_many_sequences():
    # more than 64 sequences: the scheduler kernel's chunk table
    lens = [(i * 37) % 150 for i in range(70)]
    check_bwd(custom_problem(lens, hk=2, hv=4, dk=64, dv=64, seed=210, with_state=True), 211)


def test_backward_deterministic_and_batch_invariant():
    p = custom_problem((100, 257, 64), hk=2, hv=4, dk=128, dv=128, seed=212, with_state=True)
    d_out, d_fin = upstream(p, 213)
    note("bwd: two identical calls")
    a = gpu_bwd(p, d_out, d_fin)
    b = gpu_bwd(p, d_out, d_fin)
    for name in NAMES:
        assert torch.equal(a[name], b[name]), name
    # sequence 1 alone gives the same bits as inside the batch
    cu = p.cu_seqlens.tolist()
    sl = slice(cu[1], cu[2])
    alone = Problem("alone", torch.tensor([0, cu[2] - cu[1]], dtype=torch.int32), p.q[sl].contiguous(),
                    p.k[sl].contiguous(), p.v[sl].contiguous(), p.g[sl].contiguous(), p.beta[sl].contiguous(),
                    p.state[1:2].clone())
    note("bwd: one sequence alone")
    c = gpu_bwd(alone, d_out[sl].contiguous(), d_fin[1:2].contiguous())
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(c[name], a[name][sl]), name
    assert torch.equal(c["d_init"][0], a["d_init"][1])


def test_backward_bad_cu_seqlens_writes_nothing():
    p = custom_problem((10, 20), hk=1, hv=1, dk=64, dv=64, seed=214)
    g = p.to("cuda")
    d_out, _ = upstream(p, 215, with_final=False)
    desc = la.make_desc(g.k, g.v, g.g, g.beta, 2, q=g.q, out=d_out)
    ws = torch.empty(la.la_gdn_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    for bad in ([0, 25, 20], [1, 10, 30], [0, 10, 31]):
        note(f"bwd: bad cu_seqlens {bad}")
        out = {"dq": torch.full((30, 1, 64), 3.0, device="cuda"), "dk": torch.full((30, 1, 64), 3.0, device="cuda"),
               "dv": torch.full((30, 1, 64), 3.0, device="cuda"), "dg": torch.full((30, 1), 3.0, device="cuda"),
               "dbeta": torch.full((30, 1), 3.0, device="cuda"),
               "d_initial_state": torch.full((2, 1, 64, 64), 3.0, device="cuda")}
        la.la_gdn_bwd(g.q, g.k, g.v, g.g, g.beta, torch.tensor(bad, dtype=torch.int32, device="cuda"),
                      d_out.cuda(), workspace=ws, out=out)
        assert la.la_gdn_device_status(ws) == la.LA_DEVICE_BAD_CU_SEQLENS
        for t in out.values():
            assert bool((t == 3.0).all())


def test_backward_dense_batch_slow_decay_companion():
    # the dense batch's shapes (8 x 4096 tokens, HK = 4, HV = 16, K = V = 128, initial state)
    # on its slow-decay companion, where the initial state and the gradients reach across
    # every chunk of each sequence
    check_bwd(make_problem(3, companion=True), 216)


@pytest.mark.parametrize("hk,hv", [(2, 2), (2, 4)])
def test_backward_from_the_forward_state_series_bitwise(hk, hv):
    # la_gdn_bwd_ex with the forward's fp32 series every 64 tokens: the forward's state pass is
    # skipped and every gradient equals la_gdn_bwd's bit for bit
    p = custom_problem((1, 63, 64, 65, 130, 200, 0), hk=hk, hv=hv, dk=128, dv=128, seed=219, with_state=True)
    g = p.to("cuda")
    d_out, d_fin = upstream(p, 220)
    d_out, d_fin = d_out.cuda(), d_fin.cuda()
    note(f"bwd_ex: series hk={hk} hv={hv}")
    _, _, series = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                    checkpoint_every_n_tokens=64, checkpoint_dtype=torch.float32)
    a = la.la_gdn_bwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, d_out, initial_state=g.state, d_final_state=d_fin)
    b = la.la_gdn_bwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, d_out, initial_state=g.state, d_final_state=d_fin,
                      chunk_states=series)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name


def test_backward_series_bitwise_several_rounds():
    # the varlen workload (1040 (chunk, head) items: several rounds of the backward's intra
    # workgroups, whose items also touch the cache lines of the item a round on, here in the
    # caller's series up to its last chunk): la_gdn_bwd_ex equals la_gdn_bwd bit for bit
    p = make_problem(2)
    g = p.to("cuda")
    d_out, d_fin = upstream(p, 221)
    d_out, d_fin = d_out.cuda(), d_fin.cuda()
    note("bwd_ex: series, varlen workload")
    _, _, series = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                    checkpoint_every_n_tokens=64, checkpoint_dtype=torch.float32)
    a = la.la_gdn_bwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, d_out, initial_state=g.state, d_final_state=d_fin)
    b = la.la_gdn_bwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, d_out, initial_state=g.state, d_final_state=d_fin,
                      chunk_states=series)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("hk,hv", [(2, 4), (4, 4)])
def test_backward_many_sequences_full_head_dims(hk, hv):
    # more than 64 sequences at K = V = 128 (the scheduler kernel's chunk table, the 8-wave
    # backward intra workgroup) and more (chunk, head) items than two per CU, so that the
    # intra pass runs several rounds; grouped heads (head-group sums) and one value head per
    # q/k head (the chain rule in the intra pass)
    lens = [(i * 97) % 300 for i in range(70)]
    check_bwd(custom_problem(lens, hk=hk, hv=hv, dk=128, dv=128, seed=222, with_state=True), 223)


def test_backward_two_tile_reverse_pass():
    # 5 sequences x 16 heads x 4 value tiles = 320 one-tile workgroups of the states-only
    # forward and the reverse pass, more than one per CU: both take two 32-column tiles per
    # workgroup.  A sequence alone (64 workgroups, one tile each) gives the same bits.
    p = custom_problem((130, 64, 1, 300, 77), hk=4, hv=16, dk=128, dv=128, seed=224, with_state=True)
    got, _ = check_bwd(p, 225)
    d_out, d_fin = upstream(p, 225)
    cu = p.cu_seqlens.tolist()
    for n in [0, 3]:
        sl = slice(cu[n], cu[n + 1])
        alone = Problem("alone", torch.tensor([0, cu[n + 1] - cu[n]], dtype=torch.int32), p.q[sl].contiguous(),
                        p.k[sl].contiguous(), p.v[sl].contiguous(), p.g[sl].contiguous(), p.beta[sl].contiguous(),
                        p.state[n:n + 1].clone())
        note(f"bwd: sequence {n} alone")
        c = gpu_bwd(alone, d_out[sl].contiguous(), d_fin[n:n + 1].contiguous())
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(c[name], got[name][sl]), (n, name)
        assert torch.equal(c["d_init"][0], got["d_init"][n]), n
