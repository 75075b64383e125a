"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device.

No call here reaches a HIP API: every argument set is invalid, and the checks
run first (the header states that a rejected call launches nothing).
"""
import ctypes
import os
import re

import pytest
import torch

import gated_delta_rule_50_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la_gdn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(la.LIB_PATH):
        from gated_delta_rule_50_amd import build
        build.build()
    return la.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(la.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # exported with C linkage (no mangling), checked with nm when available
    import shutil
    import subprocess
    if shutil.which("nm"):
        out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True, text=True).stdout
        syms = set(line.split()[-1] for line in out.splitlines() if line.strip())
        for name in declared_functions():
            assert name in syms, name


def _desc(N=2, T=100, HK=2, HV=4, K=128, V=128, **over):
    d = la.Desc(N, T, HK, HV, K, V, 0.0,
                HK * K, K, HK * K, K, HV * V, V, HV * V, V, HV, HV)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def test_workspace_bytes(lib):
    d = _desc()
    fwd = la.la_gdn_workspace_bytes(d, False)
    summ = la.la_gdn_workspace_bytes(d, True)
    assert fwd > 0 and summ > 0
    # per (chunk, v-head): -W (64 x K bf16), U~ (64 x V fp16), P^T (forward: six 1 KiB
    # fragments, the causal 32 x 32 tiles), per-token scalars (1 KiB)
    chunks = (100 + 63) // 64 + 2
    assert fwd >= chunks * 4 * (64 * (2 * 128 + 2 * 128) + 6 * 1024 + 1024)
    assert summ < fwd                      # no P
    bigger = la.la_gdn_workspace_bytes(_desc(T=1000), False)
    assert bigger > fwd
    assert la.la_gdn_workspace_bytes(_desc(N=0, T=0), False) > 0


@pytest.mark.parametrize("field,value,status,needle", [
    ("head_dim_k", 96, la.LA_ERR_UNSUPPORTED, "head_dim_k"),
    ("head_dim_v", 256, la.LA_ERR_UNSUPPORTED, "head_dim_v"),
    ("num_v_heads", 3, la.LA_ERR_UNSUPPORTED, "multiple"),
    ("num_qk_heads", 0, la.LA_ERR_INVALID_ARGUMENT, "num_qk_heads"),
    ("num_seqs", -1, la.LA_ERR_INVALID_ARGUMENT, "num_seqs"),
    ("total_tokens", -5, la.LA_ERR_INVALID_ARGUMENT, "total_tokens"),
])
def test_descriptor_declines(lib, field, value, status, needle):
    d = _desc(**{field: value})
    assert lib.la_gdn_workspace_bytes(ctypes.byref(d), 0) == 0
    assert needle in la.la_last_error_message()
    A = 1 << 20   # a fake, aligned address: never dereferenced because the call is rejected first
    rc = lib.la_gdn_fwd(ctypes.byref(d), A, A, A, A, A, A, None, A, A, 1, A, 1 << 30, None)
    assert rc == status
    assert needle in la.la_last_error_message()
    rc = lib.la_gdn_summary(ctypes.byref(d), A, A, A, A, A, None, A, A, 1, A, 1 << 30, None)
    assert rc == status


def _fwd_args(**over):
    A = 1 << 20
    args = dict(q=A, k=A, v=A, g=A, beta=A, cu=A, s0=None, out=A, fin=A, ws=A, wsb=1 << 30)
    args.update(over)
    return args


@pytest.mark.parametrize("over,status,needle", [
    (dict(q=None), la.LA_ERR_INVALID_ARGUMENT, "q is NULL"),
    (dict(k=(1 << 20) + 8), la.LA_ERR_INVALID_ARGUMENT, "k base pointer"),
    (dict(v=None), la.LA_ERR_INVALID_ARGUMENT, "v is NULL"),
    (dict(out=(1 << 20) + 2), la.LA_ERR_INVALID_ARGUMENT, "out base pointer"),
    (dict(g=None), la.LA_ERR_INVALID_ARGUMENT, "g is NULL"),
    (dict(beta=(1 << 20) + 1), la.LA_ERR_INVALID_ARGUMENT, "beta"),
    (dict(cu=None), la.LA_ERR_INVALID_ARGUMENT, "cu_seqlens"),
    (dict(s0=(1 << 20) + 2), la.LA_ERR_INVALID_ARGUMENT, "initial_state"),
    (dict(fin=(1 << 20) + 1), la.LA_ERR_INVALID_ARGUMENT, "final_state"),
    (dict(ws=None), la.LA_ERR_INVALID_ARGUMENT, "workspace is NULL"),
    (dict(ws=(1 << 20) + 128), la.LA_ERR_INVALID_ARGUMENT, "256-byte"),
    (dict(wsb=1024), la.LA_ERR_WORKSPACE_TOO_SMALL, "needed"),
])
def test_fwd_argument_checks(lib, over, status, needle):
    a = _fwd_args(**over)
    d = _desc()
    rc = lib.la_gdn_fwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["s0"],
                        a["out"], a["fin"], 1, a["ws"], a["wsb"], None)
    assert rc == status, la.la_last_error_message()
    assert needle in la.la_last_error_message()


@pytest.mark.parametrize("field,value,needle", [
    ("q_stride_t", 100, "q strides"),
    ("k_stride_h", 4, "k strides"),
    ("v_stride_h", 64, "head stride"),
    ("o_stride_t", 8, "overlaps"),
    ("g_stride_t", 2, "g token stride"),
])
def test_stride_checks(lib, field, value, needle):
    a = _fwd_args()
    d = _desc(**{field: value})
    rc = lib.la_gdn_fwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None,
                        a["out"], a["fin"], 1, a["ws"], a["wsb"], None)
    assert rc == la.LA_ERR_INVALID_ARGUMENT
    assert needle in la.la_last_error_message()


@pytest.mark.parametrize("field", ["q_stride_t", "k_stride_t", "v_stride_t", "g_stride_t", "beta_stride_t"])
def test_huge_token_strides_declined(lib, field):
    """Token strides of 2^24 elements or more would wrap the kernels' 32-bit offsets
    within a chunk: declined before any launch, in both calls that read the tensor."""
    a = _fwd_args()
    d = _desc(**{field: 1 << 24})
    rc = lib.la_gdn_fwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None,
                        a["out"], a["fin"], 1, a["ws"], a["wsb"], None)
    assert rc == la.LA_ERR_UNSUPPORTED, la.la_last_error_message()
    assert "2^24" in la.la_last_error_message() and field.split("_")[0] in la.la_last_error_message()
    if field != "q_stride_t":
        rc = lib.la_gdn_summary(ctypes.byref(d), a["k"], a["v"], a["g"], a["beta"], a["cu"], None, a["fin"],
                                a["out"], 1, a["ws"], a["wsb"], None)
        assert rc == la.LA_ERR_UNSUPPORTED and "2^24" in la.la_last_error_message()
    # one below the limit passes the stride checks (the call then stops at the fake workspace size)
    d = _desc(**{field: (1 << 24) - 8})
    rc = lib.la_gdn_fwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None,
                        a["out"], a["fin"], 1, a["ws"], 1024, None)
    assert rc == la.LA_ERR_WORKSPACE_TOO_SMALL, la.la_last_error_message()


def test_output_token_stride_is_not_limited(lib):
    """o rows are addressed with 64-bit offsets: a huge output stride is accepted."""
    a = _fwd_args()
    d = _desc(o_stride_t=1 << 30)
    rc = lib.la_gdn_fwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None,
                        a["out"], a["fin"], 1, a["ws"], 1024, None)
    assert rc == la.LA_ERR_WORKSPACE_TOO_SMALL, la.la_last_error_message()


def test_single_token_any_token_stride(lib):
    """With one token the token strides are never used (a broadcast view has 0): the
    checks accept them, and the library replaces them by the rows' own extents."""
    a = _fwd_args()
    d = _desc(N=1, T=1, q_stride_t=0, k_stride_t=0, v_stride_t=0, o_stride_t=0, g_stride_t=0, beta_stride_t=0)
    rc = lib.la_gdn_fwd(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None,
                        a["out"], a["fin"], 1, a["ws"], 1024, None)
    assert rc == la.LA_ERR_WORKSPACE_TOO_SMALL, la.la_last_error_message()


def test_summary_requires_outputs(lib):
    A = 1 << 20
    d = _desc()
    rc = lib.la_gdn_summary(ctypes.byref(d), A, A, A, A, A, None, None, A, 1, A, 1 << 30, None)
    assert rc == la.LA_ERR_INVALID_ARGUMENT and "end_state" in la.la_last_error_message()
    rc = lib.la_gdn_summary(ctypes.byref(d), A, A, A, A, A, None, A, None, 1, A, 1 << 30, None)
    assert rc == la.LA_ERR_INVALID_ARGUMENT and "transition" in la.la_last_error_message()


def test_empty_batch_is_a_noop(lib):
    A = 1 << 20
    d = _desc(N=0, T=0)
    rc = lib.la_gdn_fwd(ctypes.byref(d), A, A, A, A, A, A, None, A, A, 1, None, 0, None)
    assert rc == la.LA_OK


def test_binding_checks_layout():
    k = torch.zeros(10, 2, 64, dtype=torch.bfloat16)
    v = torch.zeros(10, 2, 128, dtype=torch.bfloat16).transpose(1, 2).contiguous().transpose(1, 2)
    g = torch.zeros(10, 2)
    with pytest.raises(ValueError, match="innermost"):
        la.make_desc(k, v, g, g, 1)
    d = la.make_desc(k, torch.zeros(10, 2, 128, dtype=torch.bfloat16), g, g, 1)
    assert (d.head_dim_k, d.head_dim_v, d.num_v_heads) == (64, 128, 2)


def test_profiler_ids(lib):
    names = [la.la_gdn_kernel_name(i) for i in range(la.LA_KERNEL_COUNT)]
    assert names == ["k_sched", "k_intra", "k_inter", "k_bwd_intra"]
    assert la.la_gdn_kernel_name(99) == ""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.la_gdn_profile_read(99, ctypes.byref(ms), ctypes.byref(n)) == la.LA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("fusion,beta,status,needle", [
    (dict(beta_sigmoid=0, a_log=None, dt_bias=1 << 20), 1 << 20, la.LA_ERR_INVALID_ARGUMENT, "without a_log"),
    (dict(beta_sigmoid=0, a_log=(1 << 20) + 2, dt_bias=None), 1 << 20, la.LA_ERR_INVALID_ARGUMENT, "a_log"),
    (dict(beta_sigmoid=0, a_log=1 << 20, dt_bias=(1 << 20) + 1), 1 << 20, la.LA_ERR_INVALID_ARGUMENT, "dt_bias"),
    (dict(beta_sigmoid=1, a_log=None, dt_bias=None), (1 << 20) + 1, la.LA_ERR_INVALID_ARGUMENT, "2-byte"),
    (dict(beta_sigmoid=0, a_log=None, dt_bias=None), (1 << 20) + 2, la.LA_ERR_INVALID_ARGUMENT, "4-byte"),
    (dict(beta_sigmoid=1, a_log=None, dt_bias=None), None, la.LA_ERR_INVALID_ARGUMENT, "beta is NULL"),
])
def test_fused_argument_checks(lib, fusion, beta, status, needle):
    """The gate / beta transform options are checked on the host before any launch:
    bf16 beta logits need 2-byte alignment (fp32 beta 4), a_log and dt_bias 4, and
    dt_bias only comes with a_log."""
    a = _fwd_args()
    d = _desc()
    f = la.Options(fusion["beta_sigmoid"], fusion["a_log"], fusion["dt_bias"], 0, 0, None, 0, 1)
    rc = lib.la_gdn_fwd_ex(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], beta, a["cu"], None, a["out"],
                              a["fin"], 1, ctypes.byref(f), a["ws"], a["wsb"], None)
    assert rc == status, la.la_last_error_message()
    assert needle in la.la_last_error_message()
    rc = lib.la_gdn_summary_ex(ctypes.byref(d), a["k"], a["v"], a["g"], beta, a["cu"], None, a["out"],
                                  a["fin"], 1, ctypes.byref(f), a["ws"], a["wsb"], None)
    assert rc == status, la.la_last_error_message()


def test_fused_binding_checks_beta_dtype():
    t = torch.zeros(4, 2)
    with pytest.raises(ValueError, match="bfloat16"):
        la._options(t, True, None, None)
    with pytest.raises(ValueError, match="float32"):
        la._options(t.to(torch.bfloat16), False, None, None)
    with pytest.raises(ValueError, match="a_log"):
        la._options(t, False, torch.zeros(2, dtype=torch.float64), None)


@pytest.mark.parametrize("every,cap,ck,fp32,summary,status,needle", [
    (96, 4, 1 << 20, 0, False, la.LA_ERR_UNSUPPORTED, "multiple of the 64-token chunk"),
    (-64, 4, 1 << 20, 0, False, la.LA_ERR_INVALID_ARGUMENT, "checkpoint_every_n_tokens"),
    (64, 4, None, 0, False, la.LA_ERR_INVALID_ARGUMENT, "checkpoints is NULL"),
    (64, 4, (1 << 20) + 2, 1, False, la.LA_ERR_INVALID_ARGUMENT, "4-byte"),
    (64, 4, (1 << 20) + 1, 0, False, la.LA_ERR_INVALID_ARGUMENT, "2-byte"),
    (64, -1, 1 << 20, 0, False, la.LA_ERR_INVALID_ARGUMENT, "checkpoint_capacity"),
    (64, 4, 1 << 20, 0, True, la.LA_ERR_UNSUPPORTED, "no state series"),
])
def test_checkpoint_argument_checks(lib, every, cap, ck, fp32, summary, status, needle):
    a = _fwd_args()
    d = _desc()
    o = la.Options(0, None, None, every, fp32, ck, cap, 1)
    if summary:
        rc = lib.la_gdn_summary_ex(ctypes.byref(d), a["k"], a["v"], a["g"], a["beta"], a["cu"], None, a["out"],
                                   a["fin"], 1, ctypes.byref(o), a["ws"], a["wsb"], None)
    else:
        rc = lib.la_gdn_fwd_ex(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None,
                               a["out"], a["fin"], 1, ctypes.byref(o), a["ws"], a["wsb"], None)
    assert rc == status, la.la_last_error_message()
    assert needle in la.la_last_error_message()


def test_checkpoint_entries_count():
    cu = torch.tensor([0, 1, 65, 65, 300], dtype=torch.int32)
    assert la.checkpoint_entries(cu, 64) == 1 + 1 + 0 + 4
    assert la.checkpoint_entries(cu, 128) == 1 + 1 + 0 + 2


def test_householder_options(lib):
    """Gated Delta Product: the workspace grows with the update rows, n > 64 is declined,
    and the state series is not combined with n > 1."""
    d = _desc(T=1000)
    one = la.la_gdn_workspace_bytes_ex(d, False, 1)
    assert one == la.la_gdn_workspace_bytes(d, False)
    assert la.la_gdn_workspace_bytes_ex(d, False, 3) > one
    with pytest.raises(la.LaError, match="num_householder"):
        la.la_gdn_workspace_bytes_ex(d, False, 65)
    a = _fwd_args()
    o = la.Options(0, None, None, 64, 0, 1 << 20, 4, 2)
    rc = lib.la_gdn_fwd_ex(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None, a["out"],
                           a["fin"], 1, ctypes.byref(o), a["ws"], a["wsb"], None)
    assert rc == la.LA_ERR_UNSUPPORTED and "num_householder" in la.la_last_error_message()


def _tm_options(n=2, ks=None, vs=None, bs=None, HK=2, HV=4, K=128, V=128):
    """Token-major Gated Delta Product options: update strides default to one row of heads."""
    return la.Options(0, None, None, 0, 0, None, 0, n, 1, HK * K if ks is None else ks,
                      HV * V if vs is None else vs, HV if bs is None else bs)


@pytest.mark.parametrize("desc_over,opt_over,status,needle", [
    # an update stride that is not a multiple of 8 elements
    (dict(), dict(ks=2 * 128 + 4), la.LA_ERR_INVALID_ARGUMENT, "k"),
    # updates of one token that overlap their heads
    (dict(), dict(vs=4 * 128 - 8), la.LA_ERR_INVALID_ARGUMENT, "v update stride"),
    # a token stride that does not cover the token's n update rows
    (dict(k_stride_t=2 * 128), dict(), la.LA_ERR_INVALID_ARGUMENT, "k token stride"),
    (dict(beta_stride_t=4), dict(), la.LA_ERR_INVALID_ARGUMENT, "beta token stride"),
    (dict(), dict(bs=3), la.LA_ERR_INVALID_ARGUMENT, "beta update stride"),
    # strides beyond the 32-bit offsets of one chunk's loads
    (dict(v_stride_t=1 << 23), dict(), la.LA_ERR_UNSUPPORTED, "2^23"),
])
def test_token_major_strides_checked(lib, desc_over, opt_over, status, needle):
    """Gated Delta Product, token-major k, v and beta: the token and update strides are
    checked before any launch."""
    n = 2
    base = dict(k_stride_t=n * 2 * 128, v_stride_t=n * 4 * 128, beta_stride_t=n * 4)
    base.update(desc_over)
    d = _desc(**base)
    o = _tm_options(n=n, **opt_over)
    a = _fwd_args()
    rc = lib.la_gdn_fwd_ex(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None, a["out"],
                           a["fin"], 1, ctypes.byref(o), a["ws"], a["wsb"], None)
    assert rc == status and needle in la.la_last_error_message(), la.la_last_error_message()
    rc = lib.la_gdn_summary_ex(ctypes.byref(d), a["k"], a["v"], a["g"], a["beta"], a["cu"], None, a["fin"],
                               a["out"], 1, ctypes.byref(o), a["ws"], a["wsb"], None)
    assert rc == status and needle in la.la_last_error_message(), la.la_last_error_message()


def test_token_major_descriptor_from_views():
    """make_desc and the options from rank-4 k, v and rank-3 beta views of joint
    per-token buffers: token strides in the descriptor, update strides in the options."""
    T, n, HK, HV, K, V = 5, 3, 2, 4, 64, 128
    joint = torch.zeros(T, n * HV * V + n * HK * K + 8, dtype=torch.bfloat16)
    v = joint[:, :n * HV * V].view(T, n, HV, V)
    k = joint[:, n * HV * V:n * HV * V + n * HK * K].view(T, n, HK, K)
    bj = torch.zeros(T, n * HV + 4)
    beta = bj[:, :n * HV].view(T, n, HV)
    q = torch.zeros(T, HK, K, dtype=torch.bfloat16)
    g = torch.zeros(T, HV)
    d = la.make_desc(k, v, g, beta, 1, q=q, num_householder=n)
    W = joint.stride(0)
    assert (d.total_tokens, d.num_qk_heads, d.num_v_heads, d.head_dim_k, d.head_dim_v) == (T, HK, HV, K, V)
    assert (d.k_stride_t, d.k_stride_h, d.v_stride_t, d.v_stride_h, d.beta_stride_t) == (W, K, W, V, n * HV + 4)
    o = la.Options()
    la.token_major_strides(o, k, v, beta)
    assert (o.householder_token_major, o.k_stride_update, o.v_stride_update, o.beta_stride_update) == (
        1, HK * K, HV * V, HV)
    with pytest.raises(ValueError, match="num_householder"):
        la.make_desc(k, v, g, beta, 1, q=q, num_householder=2)


def test_int64_offsets_alignment_checked(lib):
    """int64 cu_seqlens must be 8-byte aligned (int32 ones 4-byte)."""
    d = _desc()
    a = _fwd_args(cu=(1 << 20) + 4)
    o = la.Options()
    o.cu_seqlens_int64 = 1
    rc = lib.la_gdn_fwd_ex(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], None, a["out"],
                           a["fin"], 1, ctypes.byref(o), a["ws"], a["wsb"], None)
    assert rc == la.LA_ERR_INVALID_ARGUMENT and "8-byte aligned" in la.la_last_error_message()
    rc = lib.la_gdn_summary_ex(ctypes.byref(d), a["k"], a["v"], a["g"], a["beta"], a["cu"], None, a["fin"],
                               a["out"], 1, ctypes.byref(o), a["ws"], a["wsb"], None)
    assert rc == la.LA_ERR_INVALID_ARGUMENT and "8-byte aligned" in la.la_last_error_message()
    with pytest.raises(ValueError, match="int32 or int64"):
        la._cu_int64(torch.zeros(3, dtype=torch.int16))


@pytest.mark.parametrize("over,status,needle", [
    (dict(q=None), la.LA_ERR_INVALID_ARGUMENT, "q is NULL"),
    (dict(k=(1 << 20) + 8), la.LA_ERR_INVALID_ARGUMENT, "k base pointer"),
    (dict(out=(1 << 20) + 2), la.LA_ERR_INVALID_ARGUMENT, "d_out base pointer"),
    (dict(fin=None), la.LA_ERR_INVALID_ARGUMENT, "d_start_state is NULL"),
    (dict(s0=(1 << 20) + 2), la.LA_ERR_INVALID_ARGUMENT, "d_end_state"),
    (dict(wsb=1024), la.LA_ERR_WORKSPACE_TOO_SMALL, "workspace"),
])
def test_summary_bwd_argument_checks(lib, over, status, needle):
    """la_gdn_summary_bwd checks its arguments on the host before any launch."""
    d = _desc()
    a = _fwd_args(**over)
    rc = lib.la_gdn_summary_bwd(ctypes.byref(d), a["q"], a["k"], a["g"], a["beta"], a["cu"], a["out"], a["s0"],
                                a["fin"], 1, a["ws"], a["wsb"], None)
    assert rc == status and needle in la.la_last_error_message(), la.la_last_error_message()


@pytest.mark.parametrize("over,status,needle", [
    (dict(dout=None), la.LA_ERR_INVALID_ARGUMENT, "d_out is NULL"),
    (dict(dq=None), la.LA_ERR_INVALID_ARGUMENT, "dq is NULL"),
    (dict(dk=(1 << 20) + 4), la.LA_ERR_INVALID_ARGUMENT, "16-byte aligned"),
    (dict(dv=(1 << 20) + 2), la.LA_ERR_INVALID_ARGUMENT, "dv is not 4-byte"),
    (dict(dv=None), la.LA_ERR_INVALID_ARGUMENT, "dv is NULL"),
    (dict(dg=None), la.LA_ERR_INVALID_ARGUMENT, "dg is NULL"),
    (dict(dbeta=None), la.LA_ERR_INVALID_ARGUMENT, "dbeta is NULL"),
    (dict(dinit=None), la.LA_ERR_INVALID_ARGUMENT, "d_initial_state is NULL"),
    (dict(dfin=(1 << 20) + 1), la.LA_ERR_INVALID_ARGUMENT, "d_final_state"),
    (dict(ws=None), la.LA_ERR_INVALID_ARGUMENT, "workspace is NULL"),
    (dict(wsb=1024), la.LA_ERR_WORKSPACE_TOO_SMALL, "needed"),
])
def test_bwd_argument_checks(lib, over, status, needle):
    """la_gdn_bwd checks its gradients' pointers and its workspace before any launch."""
    A = 1 << 20
    a = dict(dout=A, dfin=None, dq=A, dk=A, dv=A, dg=A, dbeta=A, dinit=A, ws=A, wsb=1 << 40)
    a.update(over)
    d = _desc()
    rc = lib.la_gdn_bwd(ctypes.byref(d), A, A, A, A, A, A, None, a["dout"], a["dfin"], a["dq"], a["dk"], a["dv"],
                        a["dg"], a["dbeta"], a["dinit"], 1, a["ws"], a["wsb"], None)
    assert rc == status, la.la_last_error_message()
    assert needle in la.la_last_error_message()


def test_bwd_ex_chunk_states_checks(lib):
    """la_gdn_bwd_ex: a misaligned chunk-state series is declined before any launch; NULL
    takes la_gdn_bwd's path (the call then stops at the fake workspace's size)."""
    A = 1 << 20
    d = _desc()
    args = lambda cs, wsb: (ctypes.byref(d), A, A, A, A, A, A, None, cs, A, None, A, A, A, A, A, A, 1, A, wsb, None)
    assert lib.la_gdn_bwd_ex(*args(A + 4, 1 << 40)) == la.LA_ERR_INVALID_ARGUMENT
    assert "chunk_states" in la.la_last_error_message()
    assert lib.la_gdn_bwd_ex(*args(None, 1024)) == la.LA_ERR_WORKSPACE_TOO_SMALL
    assert lib.la_gdn_bwd_ex(*args(A, 1024)) == la.LA_ERR_WORKSPACE_TOO_SMALL


def test_bwd_workspace_bytes(lib):
    """The backward's workspace holds the forward's operands, the reverse pass's, the state
    at every chunk start and the chunk-end state gradients (fp32 K x V each per (chunk, head))."""
    d = _desc(T=1000)
    n = la.la_gdn_bwd_workspace_bytes(d)
    chunks = (1000 + 63) // 64 + 2
    assert n >= la.la_gdn_workspace_bytes(d, False) + chunks * 4 * 2 * 128 * 128 * 4
    assert lib.la_gdn_bwd_workspace_bytes(ctypes.byref(_desc(head_dim_k=96))) == 0
