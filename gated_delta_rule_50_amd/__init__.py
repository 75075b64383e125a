"""la_gdn: chunked Gated DeltaNet forward and span summary on MI355X (gfx950).

A thin ctypes binding of the C ABI declared in ``include/la_gdn.h``.  It only
marshals arguments (pointers, strides, sizes, the stream); every step of the
computation runs in the HIP kernels of ``libla_gdn.so``.  PyTorch supplies
device memory and streams.  There is no CPU fallback: if the library is not
built, importing the binding's entry points raises.

Entry points with the C names take torch tensors:
    la_gdn_fwd(q, k, v, g, beta, cu_seqlens, initial_state=None, out=None,
               final_state=None, output_final_state=True, l2norm=True, scale=None,
               workspace=None, stream=None) -> (out, final_state)
    la_gdn_summary(k, v, g, beta, cu_seqlens, start_state=None, end_state=None,
                   transition=None, l2norm=True, workspace=None, stream=None)
        -> (end_state, transition)
    la_gdn_fwd_ex(..., beta_sigmoid=False, a_log=None, dt_bias=None,
                  checkpoint_every_n_tokens=0, checkpoint_dtype=torch.bfloat16, ...)
        -> (out, final_state, checkpoints or None)
    la_gdn_summary_ex(..., beta_sigmoid=False, a_log=None, dt_bias=None, ...):
        the same with the gate / beta transforms fused into the kernels and, for the
        forward, the state series
    la_gdn_bwd(q, k, v, g, beta, cu_seqlens, d_out, initial_state=None, d_final_state=None, ...)
        -> dict of dq, dk, dv, dg, dbeta, d_initial_state (fp32): the full backward
    la_gdn_workspace_bytes(...), la_gdn_device_status(workspace),
    la_last_error_message(), la_gdn_profile_enable(on), la_gdn_profile_read(id)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libla_gdn.so")

LA_OK = 0
LA_ERR_INVALID_ARGUMENT = 1
LA_ERR_UNSUPPORTED = 2
LA_ERR_WORKSPACE_TOO_SMALL = 3
LA_ERR_HIP = 4
LA_DEVICE_OK = 0
LA_DEVICE_BAD_CU_SEQLENS = 1
LA_KERNEL_SCHED, LA_KERNEL_INTRA, LA_KERNEL_INTER, LA_KERNEL_BWD_INTRA = 0, 1, 2, 3
LA_KERNEL_COUNT = 4

# Every symbol include/la_gdn.h declares.
EXPORTED_SYMBOLS = (
    "la_gdn_workspace_bytes", "la_gdn_fwd", "la_gdn_summary", "la_gdn_fwd_ex", "la_gdn_summary_ex", "la_gdn_workspace_bytes_ex",
    "la_gdn_summary_bwd", "la_gdn_bwd_workspace_bytes", "la_gdn_bwd", "la_gdn_bwd_ex", "la_gdn_fwd_noalloc", "la_gdn_device_status",
    "la_last_error_message", "la_gdn_profile_enable", "la_gdn_profile_read", "la_gdn_kernel_name",
)


class LaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"la_gdn error {status}: {message}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("num_qk_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q_stride_t", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("k_stride_t", ctypes.c_int64), ("k_stride_h", ctypes.c_int64),
        ("v_stride_t", ctypes.c_int64), ("v_stride_h", ctypes.c_int64),
        ("o_stride_t", ctypes.c_int64), ("o_stride_h", ctypes.c_int64),
        ("g_stride_t", ctypes.c_int64), ("beta_stride_t", ctypes.c_int64),
    ]


class Options(ctypes.Structure):
    _fields_ = [
        ("beta_sigmoid", ctypes.c_int32),
        ("a_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("checkpoint_every_n_tokens", ctypes.c_int32),
        ("checkpoint_fp32", ctypes.c_int32),
        ("checkpoints", ctypes.c_void_p),
        ("checkpoint_capacity", ctypes.c_int64),
        ("num_householder", ctypes.c_int32),
        ("householder_token_major", ctypes.c_int32),
        ("k_stride_update", ctypes.c_int64),
        ("v_stride_update", ctypes.c_int64),
        ("beta_stride_update", ctypes.c_int64),
        ("cu_seqlens_int64", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libla_gdn.so.  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"la_gdn: {path} is not built; run `python -m gated_delta_rule_50_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(Desc)
    lib.la_gdn_workspace_bytes.restype = sz
    lib.la_gdn_workspace_bytes.argtypes = [dp, ctypes.c_int]
    lib.la_gdn_fwd.restype = ctypes.c_int
    lib.la_gdn_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    lib.la_gdn_summary.restype = ctypes.c_int
    lib.la_gdn_summary.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    op = ctypes.POINTER(Options)
    lib.la_gdn_workspace_bytes_ex.restype = sz
    lib.la_gdn_workspace_bytes_ex.argtypes = [dp, ctypes.c_int, op]
    lib.la_gdn_fwd_ex.restype = ctypes.c_int
    lib.la_gdn_fwd_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, op, vp, sz, vp]
    lib.la_gdn_summary_ex.restype = ctypes.c_int
    lib.la_gdn_summary_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, op, vp, sz, vp]
    lib.la_gdn_summary_bwd.restype = ctypes.c_int
    lib.la_gdn_summary_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    lib.la_gdn_bwd_workspace_bytes.restype = sz
    lib.la_gdn_bwd_workspace_bytes.argtypes = [dp]
    lib.la_gdn_bwd.restype = ctypes.c_int
    lib.la_gdn_bwd.argtypes = [dp] + [vp] * 15 + [ctypes.c_int, vp, sz, vp]
    lib.la_gdn_bwd_ex.restype = ctypes.c_int
    lib.la_gdn_bwd_ex.argtypes = [dp] + [vp] * 16 + [ctypes.c_int, vp, sz, vp]
    lib.la_gdn_fwd_noalloc.restype = ctypes.c_int
    lib.la_gdn_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    lib.la_gdn_device_status.restype = i32
    lib.la_gdn_device_status.argtypes = [vp, vp]
    lib.la_last_error_message.restype = ctypes.c_char_p
    lib.la_last_error_message.argtypes = []
    lib.la_gdn_profile_enable.restype = ctypes.c_int
    lib.la_gdn_profile_enable.argtypes = [ctypes.c_int]
    lib.la_gdn_profile_read.restype = ctypes.c_int
    lib.la_gdn_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.la_gdn_kernel_name.restype = ctypes.c_char_p
    lib.la_gdn_kernel_name.argtypes = [i32]
    _lib = lib
    return lib


def la_last_error_message() -> str:
    return load_library().la_last_error_message().decode()


def _check(status: int):
    if status != LA_OK:
        raise LaError(status, la_last_error_message())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_desc(k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              num_seqs: int, q: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              scale: Optional[float] = None, num_householder: int = 1) -> Desc:
    """Descriptor from tensor shapes and strides (no data is read).  With
    num_householder = n > 1, k, v and beta hold n update rows per token: update-major
    (k [T n, HK, K], v [T n, HV, V], beta [T n, HV]) or token-major (k [T, n, HK, K],
    v [T, n, HV, V], beta [T, n, HV]; the token strides go in the descriptor, the
    update strides in the options, see token_major_strides)."""
    tm = k.dim() == 4
    kv_rank, b_rank = (4, 3) if tm else (3, 2)
    for name, t, r in (("q", q, 3), ("k", k, kv_rank), ("v", v, kv_rank), ("out", out, 3)):
        if t is not None and (t.dim() != r or (t.shape[-1] > 1 and t.stride(-1) != 1)):
            raise ValueError(f"{name} must be rank {r} with a contiguous innermost axis")
    for name, t, r in (("g", g, 2), ("beta", beta, b_rank)):
        if t.dim() != r or (t.shape[-1] > 1 and t.stride(-1) != 1):
            raise ValueError(f"{name} must be rank {r} with a contiguous innermost axis")
    if tm:
        T, n, HK, K = k.shape
        if n != num_householder or v.shape[:2] != (T, n) or beta.shape[:2] != (T, n):
            raise ValueError("token-major k, v and beta must be [T, num_householder, ...]")
        HV, V = v.shape[2], v.shape[3]
        qq = q if q is not None else k[:, 0]
        oo = out if out is not None else v[:, 0]
        return Desc(num_seqs, T, HK, HV, K, V, float(scale) if scale else 0.0,
                    qq.stride(0), qq.stride(1), k.stride(0), k.stride(2), v.stride(0), v.stride(2),
                    oo.stride(0), oo.stride(1), g.stride(0), beta.stride(0))
    TU, HK, K = k.shape
    if TU % max(1, num_householder):
        raise ValueError("k must hold num_householder update rows per token")
    T = TU // max(1, num_householder)
    HV, V = v.shape[1], v.shape[2]
    qq = q if q is not None else k
    oo = out if out is not None else v
    return Desc(num_seqs, T, HK, HV, K, V, float(scale) if scale else 0.0,
                qq.stride(0), qq.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                oo.stride(0), oo.stride(1), g.stride(0), beta.stride(0))


def la_gdn_workspace_bytes(desc: Desc, is_summary: bool = False) -> int:
    n = load_library().la_gdn_workspace_bytes(ctypes.byref(desc), int(bool(is_summary)))
    if n == 0:
        raise LaError(LA_ERR_INVALID_ARGUMENT, la_last_error_message())
    return int(n)


def alloc_workspace(desc: Desc, is_summary: bool, device) -> torch.Tensor:
    """A workspace buffer of the right size (torch allocations are 256-byte aligned)."""
    n = la_gdn_workspace_bytes(desc, is_summary)
    return torch.empty(n, dtype=torch.uint8, device=device)


def la_gdn_fwd(q, k, v, g, beta, cu_seqlens, initial_state=None, out=None, final_state=None,
               output_final_state: bool = True, l2norm: bool = True, scale: Optional[float] = None,
               workspace: Optional[torch.Tensor] = None, stream=None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated DeltaNet forward on the GPU; returns (out, final_state or None).
    cu_seqlens is int32 or int64 (int64 goes through la_gdn_fwd_ex)."""
    if cu_seqlens.dtype == torch.int64:
        out, final_state, _ = la_gdn_fwd_ex(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                                            output_final_state, l2norm, scale, workspace=workspace,
                                            stream=stream)
        return out, final_state
    lib = load_library()
    N = cu_seqlens.numel() - 1
    T, HV, V = v.shape
    K = k.shape[2]
    if out is None:
        out = torch.empty((T, HV, V), dtype=torch.bfloat16, device=v.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, HV, K, V), dtype=torch.float32, device=v.device)
    desc = make_desc(k, v, g, beta, N, q=q, out=out, scale=scale)
    if workspace is None:
        workspace = alloc_workspace(desc, False, v.device)
    _check(lib.la_gdn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                          _ptr(cu_seqlens), _ptr(initial_state), _ptr(out), _ptr(final_state),
                          int(bool(l2norm)), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, final_state


def la_gdn_fwd_noalloc(q, k, v, g, beta, cu_seqlens, initial_state=None, out=None, final_state=None,
                       l2norm: bool = True, scale: Optional[float] = None, stream=None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """la_gdn_fwd with the library's fixed scratch array as the workspace (no device
    allocation in the call).  `out` (and `final_state`, if wanted) must be given; the
    binding allocates nothing either.  Calls that overlap on one GPU race on the array."""
    if out is None:
        raise ValueError("la_gdn_fwd_noalloc: pass out (and final_state): the call allocates nothing")
    lib = load_library()
    N = cu_seqlens.numel() - 1
    desc = make_desc(k, v, g, beta, N, q=q, out=out, scale=scale)
    _check(lib.la_gdn_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(cu_seqlens), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                  int(bool(l2norm)), _stream(stream)))
    return out, final_state


def la_gdn_summary(k, v, g, beta, cu_seqlens, start_state=None, end_state=None, transition=None,
                   l2norm: bool = True, workspace: Optional[torch.Tensor] = None, stream=None
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Span summary on the GPU; returns (end_state, transition).  cu_seqlens is int32
    or int64 (int64 goes through la_gdn_summary_ex)."""
    if cu_seqlens.dtype == torch.int64:
        return la_gdn_summary_ex(k, v, g, beta, cu_seqlens, start_state, end_state, transition, l2norm,
                                 workspace=workspace, stream=stream)
    lib = load_library()
    N = cu_seqlens.numel() - 1
    HV, V = v.shape[1], v.shape[2]
    K = k.shape[2]
    if end_state is None:
        end_state = torch.empty((N, HV, K, V), dtype=torch.float32, device=v.device)
    if transition is None:
        transition = torch.empty((N, HV, K, K), dtype=torch.float32, device=v.device)
    desc = make_desc(k, v, g, beta, N)
    if workspace is None:
        workspace = alloc_workspace(desc, True, v.device)
    _check(lib.la_gdn_summary(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                              _ptr(cu_seqlens), _ptr(start_state), _ptr(end_state), _ptr(transition),
                              int(bool(l2norm)), _ptr(workspace), workspace.numel(), _stream(stream)))
    return end_state, transition


def _options(beta: torch.Tensor, beta_sigmoid: bool, a_log, dt_bias) -> Options:
    want = torch.bfloat16 if beta_sigmoid else torch.float32
    if beta.dtype != want:
        raise ValueError(f"beta must be {want} with beta_sigmoid={beta_sigmoid}, got {beta.dtype}")
    for name, t in (("a_log", a_log), ("dt_bias", dt_bias)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 [HV] tensor")
    return Options(int(bool(beta_sigmoid)), _ptr(a_log), _ptr(dt_bias), 0, 0, None, 0, 1, 0, 0, 0, 0, 0)


def token_major_strides(opts: Options, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor):
    """Fills the token-major fields of the options from rank-4 k, v and rank-3 beta
    (no-op for update-major operands)."""
    if k.dim() == 4:
        opts.householder_token_major = 1
        opts.k_stride_update = k.stride(1)
        opts.v_stride_update = v.stride(1)
        opts.beta_stride_update = beta.stride(1)


def _cu_int64(cu_seqlens: torch.Tensor) -> int:
    if cu_seqlens.dtype not in (torch.int32, torch.int64) or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 or int64 tensor")
    return int(cu_seqlens.dtype == torch.int64)


def la_gdn_workspace_bytes_ex(desc: Desc, is_summary: bool = False, num_householder: int = 1) -> int:
    opts = Options(0, None, None, 0, 0, None, 0, int(num_householder), 0, 0, 0, 0, 0)
    n = load_library().la_gdn_workspace_bytes_ex(ctypes.byref(desc), int(bool(is_summary)), ctypes.byref(opts))
    if n == 0:
        raise LaError(LA_ERR_INVALID_ARGUMENT, la_last_error_message())
    return int(n)


def checkpoint_entries(cu_seqlens: torch.Tensor, every_n_tokens: int) -> int:
    """Entries of the state series: sum over sequences of ceil(length / n) (reads cu_seqlens)."""
    lens = (cu_seqlens[1:] - cu_seqlens[:-1]).to(torch.int64)
    return int(((lens + every_n_tokens - 1) // every_n_tokens).sum().item())


def la_gdn_fwd_ex(q, k, v, g, beta, cu_seqlens, initial_state=None, out=None, final_state=None,
                  output_final_state: bool = True, l2norm: bool = True, scale: Optional[float] = None,
                  beta_sigmoid: bool = False, a_log: Optional[torch.Tensor] = None,
                  dt_bias: Optional[torch.Tensor] = None, checkpoint_every_n_tokens: int = 0,
                  checkpoint_dtype=torch.bfloat16, checkpoints: Optional[torch.Tensor] = None,
                  num_householder: int = 1, workspace: Optional[torch.Tensor] = None, stream=None):
    """Forward with the options of la_gdn_fwd_ex: beta is bf16 logits when beta_sigmoid,
    g is the raw gate when a_log is given, and checkpoint_every_n_tokens > 0 also returns
    the state series [E, HV, K, V] (checkpoint_dtype bf16 or fp32).  Returns
    (out, final_state, checkpoints or None)."""
    lib = load_library()
    opts = _options(beta, beta_sigmoid, a_log, dt_bias)
    opts.num_householder = int(num_householder)
    token_major_strides(opts, k, v, beta)
    opts.cu_seqlens_int64 = _cu_int64(cu_seqlens)
    N = cu_seqlens.numel() - 1
    T = q.shape[0]
    HV, V = v.shape[-2], v.shape[-1]
    K = k.shape[-1]
    if out is None:
        out = torch.empty((T, HV, V), dtype=torch.bfloat16, device=v.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, HV, K, V), dtype=torch.float32, device=v.device)
    if checkpoint_every_n_tokens:
        if checkpoint_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("checkpoint_dtype must be torch.bfloat16 or torch.float32")
        if checkpoints is None:
            E = checkpoint_entries(cu_seqlens, checkpoint_every_n_tokens) if checkpoint_every_n_tokens > 0 else 0
            checkpoints = torch.empty((E, HV, K, V), dtype=checkpoint_dtype, device=v.device)
        opts.checkpoint_every_n_tokens = int(checkpoint_every_n_tokens)
        opts.checkpoint_fp32 = int(checkpoints.dtype == torch.float32)
        opts.checkpoints = _ptr(checkpoints)
        opts.checkpoint_capacity = int(checkpoints.shape[0])
    desc = make_desc(k, v, g, beta, N, q=q, out=out, scale=scale, num_householder=num_householder)
    if workspace is None:
        workspace = torch.empty(la_gdn_workspace_bytes_ex(desc, False, num_householder), dtype=torch.uint8,
                                device=v.device)
    _check(lib.la_gdn_fwd_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(cu_seqlens), _ptr(initial_state), _ptr(out), _ptr(final_state),
                             int(bool(l2norm)), ctypes.byref(opts), _ptr(workspace), workspace.numel(),
                             _stream(stream)))
    return out, final_state, checkpoints


def la_gdn_summary_ex(k, v, g, beta, cu_seqlens, start_state=None, end_state=None, transition=None,
                      l2norm: bool = True, beta_sigmoid: bool = False, a_log: Optional[torch.Tensor] = None,
                      dt_bias: Optional[torch.Tensor] = None, num_householder: int = 1,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Span summary with the gate / beta transforms fused into the kernels (and, with
    num_householder > 1, the Gated Delta Product's n update rows per token)."""
    lib = load_library()
    opts = _options(beta, beta_sigmoid, a_log, dt_bias)
    opts.num_householder = int(num_householder)
    token_major_strides(opts, k, v, beta)
    opts.cu_seqlens_int64 = _cu_int64(cu_seqlens)
    N = cu_seqlens.numel() - 1
    HV, V = v.shape[-2], v.shape[-1]
    K = k.shape[-1]
    if end_state is None:
        end_state = torch.empty((N, HV, K, V), dtype=torch.float32, device=v.device)
    if transition is None:
        transition = torch.empty((N, HV, K, K), dtype=torch.float32, device=v.device)
    desc = make_desc(k, v, g, beta, N, num_householder=num_householder)
    if workspace is None:
        workspace = torch.empty(la_gdn_workspace_bytes_ex(desc, True, num_householder), dtype=torch.uint8,
                                device=v.device)
    _check(lib.la_gdn_summary_ex(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(cu_seqlens), _ptr(start_state), _ptr(end_state), _ptr(transition),
                                 int(bool(l2norm)), ctypes.byref(opts), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    return end_state, transition


def la_gdn_summary_bwd(q, k, g, beta, cu_seqlens, d_out, d_end_state=None, d_start_state=None,
                       l2norm: bool = True, scale: Optional[float] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The span summary's mirror for the state gradient: dL/dS_start for the output
    gradients d_out [T, HV, V] (bf16) and d_end_state [N, HV, K, V] (fp32, None: zeros)."""
    lib = load_library()
    N = cu_seqlens.numel() - 1
    HV, V = d_out.shape[1], d_out.shape[2]
    K = k.shape[2]
    if d_out.dtype != torch.bfloat16 or cu_seqlens.dtype != torch.int32:
        raise ValueError("d_out must be bf16 and cu_seqlens int32")
    if d_start_state is None:
        d_start_state = torch.empty((N, HV, K, V), dtype=torch.float32, device=d_out.device)
    # the descriptor's v strides are unused here; d_out takes the o strides
    desc = make_desc(k, d_out, g, beta, N, q=q, out=d_out, scale=scale)
    if workspace is None:
        workspace = alloc_workspace(desc, True, d_out.device)
    _check(lib.la_gdn_summary_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                  _ptr(d_out), _ptr(d_end_state), _ptr(d_start_state), int(bool(l2norm)),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))
    return d_start_state


def la_gdn_bwd_workspace_bytes(desc: Desc) -> int:
    n = load_library().la_gdn_bwd_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        raise LaError(LA_ERR_INVALID_ARGUMENT, la_last_error_message())
    return int(n)


def la_gdn_bwd(q, k, v, g, beta, cu_seqlens, d_out, initial_state=None, d_final_state=None,
               l2norm: bool = True, scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
               stream=None, out: Optional[dict] = None, chunk_states: Optional[torch.Tensor] = None) -> dict:
    """Gradients of la_gdn_fwd for the upstream gradients d_out [T, HV, V] (bf16) and
    d_final_state [N, HV, K, V] (fp32, None: zeros).  Returns a dict of fp32 tensors dq, dk
    [T, HK, K], dv [T, HV, V], dg, dbeta [T, HV] and d_initial_state [N, HV, K, V] (`out`
    may hold preallocated ones).  chunk_states: the forward's fp32 state series every 64
    tokens (la_gdn_fwd_ex with checkpoint_every_n_tokens=64, checkpoint_dtype fp32), which
    spares the forward's state pass (la_gdn_bwd_ex)."""
    lib = load_library()
    if d_out.dtype != torch.bfloat16 or cu_seqlens.dtype != torch.int32 or beta.dtype != torch.float32:
        raise ValueError("d_out must be bf16, cu_seqlens int32 and beta fp32")
    N = cu_seqlens.numel() - 1
    T, HK, K = k.shape
    HV, V = v.shape[1], v.shape[2]
    dev = v.device
    shapes = {"dq": (T, HK, K), "dk": (T, HK, K), "dv": (T, HV, V), "dg": (T, HV), "dbeta": (T, HV),
              "d_initial_state": (N, HV, K, V)}
    res = dict(out or {})
    for name, shp in shapes.items():
        if name not in res:
            res[name] = torch.empty(shp, dtype=torch.float32, device=dev)
        t = res[name]
        if t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {shp}")
    desc = make_desc(k, v, g, beta, N, q=q, out=d_out, scale=scale)
    if workspace is None:
        workspace = torch.empty(la_gdn_bwd_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    grads = (_ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dg"]), _ptr(res["dbeta"]),
             _ptr(res["d_initial_state"]))
    if chunk_states is None:
        _check(lib.la_gdn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                              _ptr(initial_state), _ptr(d_out), _ptr(d_final_state), *grads, int(bool(l2norm)),
                              _ptr(workspace), workspace.numel(), _stream(stream)))
    else:
        C = checkpoint_entries(cu_seqlens, 64)
        if (chunk_states.dtype != torch.float32 or tuple(chunk_states.shape) != (C, HV, K, V)
                or not chunk_states.is_contiguous()):
            raise ValueError(f"chunk_states must be a contiguous fp32 tensor of shape {(C, HV, K, V)}")
        _check(lib.la_gdn_bwd_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(cu_seqlens), _ptr(initial_state), _ptr(chunk_states), _ptr(d_out),
                                 _ptr(d_final_state), *grads, int(bool(l2norm)), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    return res


def la_gdn_device_status(workspace: torch.Tensor, stream=None) -> int:
    return int(load_library().la_gdn_device_status(_ptr(workspace), _stream(stream)))


def la_gdn_profile_enable(enable: bool = True):
    _check(load_library().la_gdn_profile_enable(int(bool(enable))))


def la_gdn_profile_read(kernel_id: int) -> Tuple[float, int]:
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load_library().la_gdn_profile_read(kernel_id, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def la_gdn_kernel_name(kernel_id: int) -> str:
    return load_library().la_gdn_kernel_name(kernel_id).decode()
