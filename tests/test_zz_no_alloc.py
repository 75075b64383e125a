"""GPU: la_gdn_fwd_noalloc, the forward with the library's fixed scratch array as its
workspace, called through the C ABI, against la_gdn_fwd with a workspace of its own:
equal bit for bit (the same kernels on the same inputs) and within the oracle's
tolerances, on two calls in a row, the second one smaller than the first (the array
keeps the first call's contents).  A problem whose workspace exceeds the array is
declined before any launch."""
import pytest
import torch

import gated_delta_rule_50_amd as la
from oracle import Oracle
from workloads import custom_problem, make_problem

from gpu_helpers import assert_o_state, gpu_fwd, note

pytestmark = pytest.mark.gpu


def test_noalloc_equals_fwd_on_two_calls_in_a_row():
    for p in (make_problem(2), custom_problem((100, 37, 300), hk=2, hv=4, dk=128, dv=64, seed=61,
                                              with_state=True)):
        note(f"noalloc: {p.name}")
        out_ref, fin_ref = gpu_fwd(p)
        g = p.to("cuda")
        out = torch.empty_like(out_ref)
        fin = torch.empty_like(fin_ref)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        la.la_gdn_fwd_noalloc(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state, out=out,
                              final_state=fin)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(out, out_ref) and torch.equal(fin, fin_ref)
        assert_o_state(out, fin, Oracle(p).run_all())


def test_noalloc_declines_a_problem_beyond_the_scratch_array():
    T, H, D = 8192, 32, 128
    q = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    gb = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    note("noalloc: too large")
    with pytest.raises(la.LaError, match="scratch") as e:
        la.la_gdn_fwd_noalloc(q, q, q, gb, gb, cu, out=out)
    assert e.value.status == la.LA_ERR_WORKSPACE_TOO_SMALL
