"""The extended calls with more than 64 sequences, where the scheduler kernel
(k_sched) builds the chunk table: the Gated Delta Product's update rows, the
state series' per-sequence entry offsets and the fused gate and beta, against
the fp64 oracle.  Lengths include empty and one-token sequences."""
import numpy as np
import pytest
import torch

import gated_delta_rule_50_amd as la
from oracle import Oracle, rel_l2
from workloads import custom_problem, fused_problem, gdp_problem

from gpu_helpers import TOL_O, TOL_STATE, assert_o_state, assert_states, f64, note

pytestmark = pytest.mark.gpu

LENGTHS = tuple([0, 1, 2, 63, 64, 65] + [(7 * i) % 90 for i in range(64)])   # 70 sequences


def test_gdp_many_sequences():
    p = gdp_problem(LENGTHS, 2, hk=1, hv=2, dk=64, dv=64, seed=101, with_state=True)
    g = p.to("cuda")
    note(f"gdp n=2, {p.num_seqs} sequences")
    out, fin, _ = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                   num_householder=2)
    torch.cuda.synchronize()
    ref = Oracle(p).run_all()
    assert_o_state(out, fin, ref)


def test_series_many_sequences():
    p = custom_problem(LENGTHS, hk=1, hv=2, dk=64, dv=64, seed=102, with_state=True)
    g = p.to("cuda")
    note(f"series, {p.num_seqs} sequences")
    out, fin, ck = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                    checkpoint_every_n_tokens=64, checkpoint_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = Oracle(p).run_all(checkpoint_every=64)
    assert ck.shape[0] == ref["checkpoints"].shape[0]
    assert_states(ck, ref["checkpoints"], TOL_STATE, "state series")
    assert_o_state(out, None, ref)


def test_fused_many_sequences():
    p = fused_problem(LENGTHS, hk=1, hv=2, dk=64, dv=64, seed=103, with_state=True)
    g = p.to("cuda")
    note(f"fused gate and beta, {p.num_seqs} sequences")
    out, fin, _ = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                   beta_sigmoid=True, a_log=g.a_log, dt_bias=g.dt_bias)
    torch.cuda.synchronize()
    ref = Oracle(p).run_all()
    assert_o_state(out, fin, ref)
