"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: rel-L2 <= 1e-2 for the bf16 output o and <= 5e-3 for fp32 final
states, end states and transitions, over the whole tensor and, within five
times that, row by row (one token-head of o, one (sequence, head) state or
transition).  Every element of every workload is compared, the long-context
and span workloads unit by unit, plus properties that hold at any size.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_50_amd as la
from oracle import Oracle, rel_l2
from workloads import Problem, custom_problem, make_problem

from gpu_helpers import (TOL_O, TOL_STATE, UnitTally, assert_o_state, assert_rows_close, assert_summary,
                         check_fwd_full, f64, gpu_fwd, gpu_summary, note)

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------
# small and medium shapes: every element

@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_ragged_small_all_head_dims(dk, dv):
    # several chunks, ragged tails, a length-1 and an exact-chunk sequence
    p = custom_problem((1, 63, 64, 65, 130, 200), hk=2, hv=4, dk=dk, dv=dv, seed=21, with_state=True)
    check_fwd_full(p)


def test_config1_tiny():
    check_fwd_full(make_problem(1))


def test_config2_varlen():
    check_fwd_full(make_problem(2))


def test_no_l2norm_custom_scale():
    p = custom_problem((70, 130), hk=1, hv=2, dk=64, dv=64, seed=22, l2norm=False, with_state=True)
    # without the norm, |k|^2 ~ 64: shrink k so the recurrence stays contractive
    p = dataclasses.replace(p, k=(p.k.float() / 8).to(torch.bfloat16), q=(p.q.float() / 8).to(torch.bfloat16))
    note("no l2norm, scale 0.3")
    out, fin = gpu_fwd(p, scale=0.3)
    ref = Oracle(p, scale=0.3).run_all()
    assert_o_state(out, fin, ref)


def test_summary_small_slow_decay():
    p = custom_problem((1, 64, 100, 300), hk=2, hv=2, dk=128, dv=128, seed=23, with_state=True,
                       summary=True, g_div=4096.0, beta_div=64.0)
    note("summary small slow decay")
    end, tr = gpu_summary(p)
    ref = Oracle(p).run_all(want_o=False, want_transition=True)
    assert_summary(end, tr, ref)
    assert np.abs(ref["transition"]).max() > 0.05   # not vacuous


def test_summary_small_k64():
    p = custom_problem((37, 64, 129), hk=1, hv=3, dk=64, dv=128, seed=24, with_state=True,
                       summary=True, g_div=512.0, beta_div=8.0)
    note("summary K=64 V=128")
    end, tr = gpu_summary(p)
    ref = Oracle(p).run_all(want_o=False, want_transition=True)
    assert_summary(end, tr, ref)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_summary_two_tile_workgroups_all_head_dims(dk, dv):
    # 70 spans x 2 heads x (K + V) / 32 tiles: more than two one-tile workgroups per CU, so
    # the summary runs two 32-column tiles per workgroup (S and P column pairs)
    lengths = [(i * 53) % 200 for i in range(70)]
    p = custom_problem(lengths, hk=1, hv=2, dk=dk, dv=dv, seed=26, with_state=True, summary=True,
                       g_div=512.0, beta_div=8.0)
    note(f"summary two-tile workgroups K={dk} V={dv}")
    end, tr = gpu_summary(p)
    ref = Oracle(p).run_all(want_o=False, want_transition=True)
    assert_summary(end, tr, ref)
    # a span alone runs the one-tile workgroups: the same bits
    cu = p.cu_seqlens.tolist()
    for n in [1, 7, 69]:
        sl = slice(cu[n], cu[n + 1])
        alone = dataclasses.replace(p, name="alone", cu_seqlens=torch.tensor([0, cu[n + 1] - cu[n]], dtype=torch.int32),
                                    k=p.k[sl].contiguous(), v=p.v[sl].contiguous(), g=p.g[sl].contiguous(),
                                    beta=p.beta[sl].contiguous(), state=p.state[n:n + 1].clone())
        ea, ta = gpu_summary(alone)
        assert torch.equal(ea[0], end[n]) and torch.equal(ta[0], tr[n]), n


def test_empty_sequences_and_identity_transition():
    p = custom_problem((0, 5, 0, 70, 0), hk=1, hv=2, dk=64, dv=64, seed=25, with_state=True)
    note("empty sequences fwd")
    out, fin = gpu_fwd(p)
    ref = Oracle(p).run_all()
    assert_o_state(out, fin, ref)
    for n in (0, 2, 4):
        assert torch.equal(fin[n].cpu(), p.state[n])
    ps = dataclasses.replace(p, q=None, summary=True)
    note("empty sequences summary")
    end, tr = gpu_summary(ps)
    for n in (0, 2, 4):
        assert torch.equal(end[n].cpu(), p.state[n])
        assert torch.equal(tr[n].cpu(), torch.eye(64).expand(2, 64, 64))


# ----------------------------------------------------------------------------
# the five workloads

def test_config3_grouped_heads_initial_state():
    p = make_problem(3)
    out, fin, ref, eo, es = check_fwd_full(p)
    # the initial state barely reaches o under this gate; check the first chunk alone
    first = np.concatenate([np.arange(n * 4096, n * 4096 + 64) for n in range(8)])
    e1 = rel_l2(f64(out)[first], ref["o"][first])
    assert e1 <= TOL_O, e1
    assert_rows_close(f64(out)[first], ref["o"][first], TOL_O, "first-chunk o rows")


def test_config3_slow_decay_companion():
    p = make_problem(3, companion=True)
    out, fin, ref, eo, es = check_fwd_full(p)
    # dropping the initial state would move o by far more than the tolerance here
    no_s0 = Oracle(p, use_initial_state=False).run_units([(0, 0)])["o"][0]
    assert rel_l2(no_s0, ref["o"][:4096, 0]) > 0.1


def _all_units_longest_first(o: Oracle):
    units = o.all_units()
    lens = o.lengths()
    units.sort(key=lambda u: -lens[u[0]])
    return units


def test_config4_ragged_long_context_every_unit():
    """Every one of the 65 x 32 (sequence, head) units against the oracle: each unit's o
    and final state within the tolerance on its own (so that a short sequence cannot
    hide under the 65536-token one), the whole tensors, and every row."""
    p = make_problem(4)
    note(f"config 4 T={p.total_tokens}")
    out, fin = gpu_fwd(p, initial_state=False)
    orc = Oracle(p, use_initial_state=False)
    units = _all_units_longest_first(orc)
    note(f"config 4 oracle over {len(units)} units")
    ref = orc.run_units(units, want_o=True)
    cu = p.cu_seqlens.tolist()
    out_c, fin_c = out.cpu(), fin.cpu()
    to, ts = UnitTally(TOL_O, "o"), UnitTally(TOL_STATE, "final state")
    for (n, h), ro, rs in zip(units, ref["o"], ref["state"]):
        to.add(out_c[cu[n]:cu[n + 1], h].double().numpy(), ro, (n, h))
        ts.add(fin_c[n, h].double().numpy().reshape(1, -1), rs.reshape(1, -1), (n, h))
    print(f"config 4: o rel-L2 {to.check():.3e}, final state rel-L2 {ts.check():.3e}", flush=True)


def test_config5_summary_every_unit():
    """All 32 x 16 units of the span summary.  Under this gate the exact transition
    underflows to 0 even in fp64 (e^(sum g) over 8192 tokens), so the transition is
    checked to be 0 here and compared in earnest on the slow-decay companion below."""
    p = make_problem(5)
    note(f"config 5 T={p.total_tokens}")
    end, tr = gpu_summary(p)
    orc = Oracle(p)
    units = _all_units_longest_first(orc)
    note(f"config 5 oracle over {len(units)} units")
    ref = orc.run_units(units, want_o=False, want_transition=True)
    end_c, tr_c = end.cpu(), tr.cpu()
    te = UnitTally(TOL_STATE, "end state")
    for (n, h), rs, rt in zip(units, ref["state"], ref["transition"]):
        te.add(end_c[n, h].double().numpy().reshape(1, -1), rs.reshape(1, -1), (n, h))
        assert np.abs(rt).max() <= 1e-30
        assert float(tr_c[n, h].abs().max()) <= 1e-30, (n, h)
    print(f"config 5: end state rel-L2 {te.check():.3e}", flush=True)


def test_config5_companion_summary_and_composition():
    """Slow-decay companion: every unit's end state and transition against the oracle,
    and the fold of all 32 span summaries against one forward pass over the
    concatenated spans."""
    p = make_problem(5, companion=True)
    note("config 5 companion summary")
    end, tr = gpu_summary(p)
    orc = Oracle(p)
    units = _all_units_longest_first(orc)
    note(f"config 5 companion oracle over {len(units)} units")
    ref = orc.run_units(units, want_o=False, want_transition=True)
    end_c, tr_c = end.cpu(), tr.cpu()
    te, tt = UnitTally(TOL_STATE, "end state"), UnitTally(TOL_STATE, "transition")
    for (n, h), rs, rt in zip(units, ref["state"], ref["transition"]):
        te.add(end_c[n, h].double().numpy().reshape(1, -1), rs.reshape(1, -1), (n, h))
        tt.add(tr_c[n, h].double().numpy().reshape(1, -1), rt.reshape(1, -1), (n, h))
    print(f"config 5': end state rel-L2 {te.check():.3e}, transition rel-L2 {tt.check():.3e}", flush=True)
    assert max(float(np.abs(rt).max()) for rt in ref["transition"]) > 0.05   # not vacuous
    # zero-start spans, folded with the transitions
    note("config 5 companion zero-start summary + fold")
    span_end, span_tr = gpu_summary(p, start_state=False)
    X = p.state[0].double().cuda()                      # [HV, K, V]
    for i in range(32):
        X = torch.einsum("hiv,hij->hjv", X, span_tr[i].double()) + span_end[i].double()
    # one sequence over all 262144 tokens, started from span 0's start state
    whole = dataclasses.replace(p, cu_seqlens=torch.tensor([0, p.total_tokens], dtype=torch.int32),
                                state=p.state[:1].clone(), q=p.k.clone(), summary=False)
    note("config 5 companion unsplit forward")
    _, fin = gpu_fwd(whole)
    assert rel_l2(f64(X), f64(fin[0])) <= TOL_STATE
    assert_rows_close(f64(X).reshape(16, -1), f64(fin[0]).reshape(16, -1), TOL_STATE, "folded states")


# ----------------------------------------------------------------------------
# invariants on the GPU

def test_batch_invariance_bitwise_config4():
    p = make_problem(4)
    note("config 4 batch invariance")
    out, fin = gpu_fwd(p, initial_state=False)
    cu = p.cu_seqlens.tolist()
    N = len(cu) - 1
    for n in [0, 1, 2, 17, N - 1]:
        sl = slice(cu[n], cu[n + 1])
        alone = Problem("alone", torch.tensor([0, cu[n + 1] - cu[n]], dtype=torch.int32),
                        p.q[sl].contiguous(), p.k[sl].contiguous(), p.v[sl].contiguous(),
                        p.g[sl].contiguous(), p.beta[sl].contiguous(), None)
        oa, fa = gpu_fwd(alone, initial_state=False)
        assert torch.equal(oa, out[sl]), n
        assert torch.equal(fa[0], fin[n]), n
    # a permuted batch: long sequence first, then the rest reversed
    perm = [N - 1] + list(range(N - 2, -1, -1))
    parts = [slice(cu[n], cu[n + 1]) for n in perm]
    lens = [cu[n + 1] - cu[n] for n in perm]
    cu2 = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    cat = lambda t: torch.cat([t[s] for s in parts]).contiguous()
    pp = Problem("perm", cu2, cat(p.q), cat(p.k), cat(p.v), cat(p.g), cat(p.beta), None)
    note("config 4 permuted batch")
    op, fp = gpu_fwd(pp, initial_state=False)
    for j, n in enumerate(perm):
        assert torch.equal(op[cu2[j]:cu2[j + 1]], out[cu[n]:cu[n + 1]]), n
        assert torch.equal(fp[j], fin[n]), n


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_two_tile_inter_pass_equals_one_tile_bitwise(dk, dv):
    # 40 sequences, 2 (V = 128) or 4 (V = 64) value heads: 320 one-tile inter workgroups, more
    # than the 256 CUs and at most twice as many, so the batch runs the two-tile inter
    # kernel; each sequence alone runs the one-tile one.  Same bits, and the batch within the
    # tolerances of the oracle.
    lens = [(i * 53) % 300 + 1 for i in range(40)]
    hv = 2 if dv == 128 else 4
    p = custom_problem(lens, hk=hv // 2, hv=hv, dk=dk, dv=dv, seed=27, with_state=True)
    note(f"two-tile inter pass dk={dk} dv={dv}")
    out, fin = check_fwd_full(p)[:2]
    cu = p.cu_seqlens.tolist()
    for n in [0, 7, 39]:
        sl = slice(cu[n], cu[n + 1])
        alone = Problem("alone", torch.tensor([0, cu[n + 1] - cu[n]], dtype=torch.int32),
                        p.q[sl].contiguous(), p.k[sl].contiguous(), p.v[sl].contiguous(),
                        p.g[sl].contiguous(), p.beta[sl].contiguous(), p.state[n:n + 1].clone())
        oa, fa = gpu_fwd(alone)
        assert torch.equal(oa, out[sl]), n
        assert torch.equal(fa[0], fin[n]), n


def test_repeat_calls_bitwise_identical():
    p = make_problem(2)
    note("repeat calls")
    o1, f1 = gpu_fwd(p)
    o2, f2 = gpu_fwd(p)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_grouped_heads_equal_duplicated_heads_bitwise():
    p = custom_problem((100, 257), hk=2, hv=8, dk=128, dv=128, seed=26, with_state=True)
    rep = torch.arange(8) // 4
    dup = dataclasses.replace(p, q=p.q[:, rep].contiguous(), k=p.k[:, rep].contiguous())
    note("grouped vs duplicated heads")
    o1, f1 = gpu_fwd(p)
    o2, f2 = gpu_fwd(dup)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_strided_views_of_fused_projection():
    """q, k, v as column slices of one [T, (2 HK K + HV V)] projection, o into a
    wider buffer: the same bits as contiguous inputs."""
    p = custom_problem((90, 200), hk=2, hv=4, dk=64, dv=128, seed=27, with_state=True)
    T = p.total_tokens
    fused = torch.cat([p.q.reshape(T, -1), p.k.reshape(T, -1), p.v.reshape(T, -1)], dim=1).cuda()
    q = fused[:, :128].view(T, 2, 64)
    k = fused[:, 128:256].view(T, 2, 64)
    v = fused[:, 256:].view(T, 4, 128)
    gbuf = torch.zeros(T, 12).cuda()
    gbuf[:, 4:8] = p.g.cuda()
    g = gbuf[:, 4:8]
    obuf = torch.zeros(T, 4, 256, dtype=torch.bfloat16, device="cuda")
    out = obuf[:, :, 64:192]
    note("strided views")
    la.la_gdn_fwd(q, k, v, g, p.beta.cuda(), p.cu_seqlens.cuda(), initial_state=p.state.cuda(), out=out)
    o_ref, f_ref = gpu_fwd(p)
    assert torch.equal(out, o_ref)
    assert torch.equal(obuf[:, :, :64], torch.zeros_like(obuf[:, :, :64]))


def test_bad_cu_seqlens_sets_status_and_writes_nothing():
    p = custom_problem((10, 20), hk=1, hv=1, dk=64, dv=64, seed=28)
    g = p.to("cuda")
    desc = la.make_desc(g.k, g.v, g.g, g.beta, 2, q=g.q)
    ws = la.alloc_workspace(desc, False, "cuda")
    for bad in ([0, 25, 20], [1, 10, 30], [0, 10, 31], [0, -1, 30]):
        note(f"bad cu_seqlens {bad}")
        out = torch.full((30, 1, 64), 7.0, dtype=torch.bfloat16, device="cuda")
        fin = torch.full((2, 1, 64, 64), 3.0, device="cuda")
        la.la_gdn_fwd(g.q, g.k, g.v, g.g, g.beta, torch.tensor(bad, dtype=torch.int32, device="cuda"),
                      out=out, final_state=fin, workspace=ws)
        assert la.la_gdn_device_status(ws) == la.LA_DEVICE_BAD_CU_SEQLENS
        assert bool((out == 7.0).all()) and bool((fin == 3.0).all())
    la.la_gdn_fwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, workspace=ws)
    assert la.la_gdn_device_status(ws) == la.LA_DEVICE_OK


def test_final_state_null_and_chaining():
    """final_state -> initial_state round trip over a split at 64 and at 37."""
    p = custom_problem((300,), hk=2, hv=2, dk=128, dv=128, seed=29, with_state=True, g_div=64.0)
    o_full, f_full = gpu_fwd(p)
    for split in (64, 37):
        a = Problem("a", torch.tensor([0, split], dtype=torch.int32), p.q[:split], p.k[:split],
                    p.v[:split], p.g[:split], p.beta[:split], p.state)
        oa, fa = gpu_fwd(a)
        b = Problem("b", torch.tensor([0, 300 - split], dtype=torch.int32), p.q[split:].contiguous(),
                    p.k[split:].contiguous(), p.v[split:].contiguous(), p.g[split:].contiguous(),
                    p.beta[split:].contiguous(), fa.cpu())
        ob, fb = gpu_fwd(b)
        ref = Oracle(p).run_all()
        assert rel_l2(f64(torch.cat([oa, ob])), ref["o"]) <= TOL_O
        assert rel_l2(f64(fb), ref["state"]) <= TOL_STATE
        assert_o_state(torch.cat([oa, ob]), fb, ref)
    g = p.to("cuda")
    out, fin = la.la_gdn_fwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                             output_final_state=False)
    assert fin is None and torch.equal(out, o_full)


def test_single_token_with_zero_token_strides():
    """One token given as broadcast views (token stride 0) for every operand, and the
    output written through a stride-0 view: the same bits as contiguous tensors, and the
    oracle's values (a single-token decode step)."""
    p = custom_problem((1,), hk=2, hv=4, dk=128, dv=128, seed=30, with_state=True)
    g = p.to("cuda")

    def zero_t(t):
        return torch.as_strided(t, t.shape, (0,) + tuple(t.stride()[1:]))

    out = torch.empty((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    note("single token, token strides 0")
    o0, f0 = la.la_gdn_fwd(zero_t(g.q), zero_t(g.k), zero_t(g.v), zero_t(g.g), zero_t(g.beta), g.cu_seqlens,
                           initial_state=g.state, out=zero_t(out))
    o1, f1 = gpu_fwd(p)
    assert torch.equal(o0, o1) and torch.equal(f0, f1)
    assert_o_state(o0, f0, Oracle(p).run_all())
    end0, tr0 = la.la_gdn_summary(zero_t(g.k), zero_t(g.v), zero_t(g.g), zero_t(g.beta), g.cu_seqlens,
                                  start_state=g.state)
    end1, tr1 = gpu_summary(dataclasses.replace(p, q=None, summary=True))
    torch.cuda.synchronize()
    assert torch.equal(end0, end1) and torch.equal(tr0, tr1)
