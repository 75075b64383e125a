"""The compute calls under HIP graph capture (torch.cuda.CUDAGraph): the library
enqueues only kernels on the caller's stream (no memsets, no host syncs, no
allocations), so a captured forward or summary replays on new inputs.  Each of
several replays, with eager work and synchronisations between them, must equal
an eager call on the same inputs bit for bit."""
import pytest
import torch

import gated_delta_rule_50_amd as la
from workloads import make_problem, custom_problem

from gpu_helpers import note

pytestmark = pytest.mark.gpu


def _load(dst, src):
    for name in ("q", "k", "v", "g", "beta", "state"):
        a, b = getattr(dst, name), getattr(src, name)
        if a is not None:
            a.copy_(b)


def test_forward_graph_replays_match_eager():
    p = make_problem(2).to("cuda")
    T, HV, V, K, N = p.total_tokens, p.num_v_heads, p.head_dim_v, p.head_dim_k, p.num_seqs
    out = torch.empty((T, HV, V), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((N, HV, K, V), dtype=torch.float32, device="cuda")
    ws = la.alloc_workspace(la.make_desc(p.k, p.v, p.g, p.beta, N, q=p.q, out=out), False, "cuda")

    def call():
        la.la_gdn_fwd(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, out=out, final_state=fin, workspace=ws)

    call()
    torch.cuda.synchronize()
    note("graph capture of la_gdn_fwd")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        _load(p, make_problem(2, seed=300 + rep).to("cuda"))
        graph.replay()
        torch.cuda.synchronize()
        o_g, f_g = out.clone(), fin.clone()
        o_e, f_e = la.la_gdn_fwd(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens)   # eager, fresh buffers
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(f_g, f_e), f"replay {rep}"


def test_summary_graph_replays_match_eager():
    p = custom_problem((100, 300, 64), hk=2, hv=2, dk=128, dv=128, seed=310, with_state=True,
                       summary=True, g_div=4096.0, beta_div=64.0).to("cuda")
    N, HV, K, V = p.num_seqs, p.num_v_heads, p.head_dim_k, p.head_dim_v
    end = torch.empty((N, HV, K, V), dtype=torch.float32, device="cuda")
    tr = torch.empty((N, HV, K, K), dtype=torch.float32, device="cuda")
    ws = la.alloc_workspace(la.make_desc(p.k, p.v, p.g, p.beta, N), True, "cuda")

    def call():
        la.la_gdn_summary(p.k, p.v, p.g, p.beta, p.cu_seqlens, start_state=p.state, end_state=end,
                          transition=tr, workspace=ws)

    call()
    torch.cuda.synchronize()
    note("graph capture of la_gdn_summary")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        _load(p, custom_problem((100, 300, 64), hk=2, hv=2, dk=128, dv=128, seed=320 + rep, with_state=True,
                                summary=True, g_div=4096.0, beta_div=64.0).to("cuda"))
        graph.replay()
        torch.cuda.synchronize()
        e_g, t_g = end.clone(), tr.clone()
        e_e, t_e = la.la_gdn_summary(p.k, p.v, p.g, p.beta, p.cu_seqlens, start_state=p.state)
        torch.cuda.synchronize()
        assert torch.equal(e_g, e_e) and torch.equal(t_g, t_e), f"replay {rep}"


def test_summary_bwd_and_int64_offsets_graph_replays_match_eager():
    """la_gdn_summary_bwd, and the forward with int64 cu_seqlens (its conversion kernel
    included), captured and replayed on new inputs."""
    lengths = (100, 0, 300, 64)
    p = custom_problem(lengths, hk=2, hv=4, dk=128, dv=64, seed=330, with_state=True).to("cuda")
    N, HV, K, V, T = p.num_seqs, p.num_v_heads, p.head_dim_k, p.head_dim_v, p.total_tokens
    gen = torch.Generator(device="cuda").manual_seed(331)
    d_out = torch.randn((T, HV, V), generator=gen, device="cuda").to(torch.bfloat16)
    d_end = torch.randn((N, HV, K, V), generator=gen, device="cuda")
    d_start = torch.empty((N, HV, K, V), dtype=torch.float32, device="cuda")
    cu64 = p.cu_seqlens.to(torch.int64)
    out = torch.empty((T, HV, V), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((N, HV, K, V), dtype=torch.float32, device="cuda")
    desc = la.make_desc(p.k, p.v, p.g, p.beta, N, q=p.q, out=out)
    ws_b = la.alloc_workspace(desc, True, "cuda")
    ws_f = la.alloc_workspace(desc, False, "cuda")

    def call():
        la.la_gdn_summary_bwd(p.q, p.k, p.g, p.beta, p.cu_seqlens, d_out, d_end, d_start_state=d_start,
                              workspace=ws_b)
        la.la_gdn_fwd(p.q, p.k, p.v, p.g, p.beta, cu64, initial_state=p.state, out=out, final_state=fin,
                      workspace=ws_f)

    call()
    torch.cuda.synchronize()
    note("graph capture of la_gdn_summary_bwd and la_gdn_fwd with int64 offsets")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        _load(p, custom_problem(lengths, hk=2, hv=4, dk=128, dv=64, seed=340 + rep, with_state=True).to("cuda"))
        d_out.copy_(torch.randn((T, HV, V), generator=gen, device="cuda").to(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        s_g, o_g, f_g = d_start.clone(), out.clone(), fin.clone()
        s_e = la.la_gdn_summary_bwd(p.q, p.k, p.g, p.beta, p.cu_seqlens, d_out, d_end)
        o_e, f_e = la.la_gdn_fwd(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, initial_state=p.state)
        torch.cuda.synchronize()
        assert torch.equal(s_g, s_e) and torch.equal(o_g, o_e) and torch.equal(f_g, f_e), f"replay {rep}"


def test_backward_graph_replays_match_eager():
    p = custom_problem((100, 257, 64), hk=2, hv=4, dk=128, dv=128, seed=330, with_state=True).to("cuda")
    T, HK, HV, K, V, N = p.total_tokens, p.num_qk_heads, p.num_v_heads, p.head_dim_k, p.head_dim_v, p.num_seqs
    gen = torch.Generator(device="cuda").manual_seed(331)
    d_out = torch.randn((T, HV, V), generator=gen, device="cuda").to(torch.bfloat16)
    d_fin = torch.randn((N, HV, K, V), generator=gen, device="cuda")
    grads = {"dq": torch.empty((T, HK, K), device="cuda"), "dk": torch.empty((T, HK, K), device="cuda"),
             "dv": torch.empty((T, HV, V), device="cuda"), "dg": torch.empty((T, HV), device="cuda"),
             "dbeta": torch.empty((T, HV), device="cuda"), "d_initial_state": torch.empty((N, HV, K, V), device="cuda")}
    desc = la.make_desc(p.k, p.v, p.g, p.beta, N, q=p.q, out=d_out)
    ws = torch.empty(la.la_gdn_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")

    def call():
        la.la_gdn_bwd(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, d_out, initial_state=p.state, d_final_state=d_fin,
                      workspace=ws, out=grads)

    call()
    torch.cuda.synchronize()
    note("graph capture of la_gdn_bwd")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        _load(p, custom_problem((100, 257, 64), hk=2, hv=4, dk=128, dv=128, seed=332 + rep,
                                with_state=True).to("cuda"))
        d_out.copy_(torch.randn((T, HV, V), generator=gen, device="cuda").to(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        got = {k: t.clone() for k, t in grads.items()}
        eager = la.la_gdn_bwd(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, d_out, initial_state=p.state,
                              d_final_state=d_fin)
        torch.cuda.synchronize()
        for k in got:
            assert torch.equal(got[k], eager[k]), f"replay {rep}: {k}"
