"""fp64 CPU oracle for the Gated DeltaNet forward, span summary and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The GPU library
never loads it and shares no code with it.

The arithmetic lives in ``gdn_oracle.c`` (plain token-by-token recurrence in
double precision; see the comment at its top for the definition and the
passages of the pages it follows).  This module builds that file with gcc,
binds it with ctypes and arranges inputs and outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")

_lib = None


def build() -> str:
    """Compile the oracle with gcc (fp64, no fast-math, OpenMP)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_qk_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("l2norm", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("cu_seqlens", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p),
        ("beta_logit", ctypes.c_void_p),
        ("a_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("checkpoint_every", ctypes.c_int32),
        ("checkpoints", ctypes.c_void_p),
        ("checkpoint_offset", ctypes.c_void_p),
        ("num_householder", ctypes.c_int32),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.gdn_oracle_run.restype = ctypes.c_int
        lib.gdn_oracle_run.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.gdn_oracle_backward.restype = ctypes.c_int
        lib.gdn_oracle_backward.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32] + [ctypes.c_void_p] * 11 + [
            ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    """Threads for the oracle: the CPUs this process may use, at most OMP_NUM_THREADS
    and at most 16, the host's CPU share of one GPU on an MI355X node (the benchmark
    reports the host's CPU count and model beside the figure)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, min(n, 16))


def _ptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _bits(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    if t is None:
        return None
    assert t.dtype == torch.bfloat16
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy()).view(np.uint16)


def _f32(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    if t is None:
        return None
    return np.ascontiguousarray(t.detach().cpu().to(torch.float32).numpy())


class Oracle:
    """Binds one problem's host tensors to the C oracle.

    ``problem`` is a ``workloads.Problem`` (or any object with the same
    fields).  ``scale=None`` means K^-1/2.
    """

    def __init__(self, problem, scale: Optional[float] = None, initial_state=None,
                 use_initial_state: bool = True):
        p = problem
        self.cu = np.ascontiguousarray(p.cu_seqlens.detach().cpu().to(torch.int32).numpy())
        self.q = _bits(p.q)
        self.k = _bits(p.k)
        self.v = _bits(p.v)
        self.g = _f32(p.g)
        # gate and beta transforms: a problem with beta_sigmoid carries bf16 beta logits;
        # one with a_log carries the raw gate (see gdn_oracle.c)
        fused_beta = bool(getattr(p, "beta_sigmoid", False))
        self.beta = None if fused_beta else _f32(p.beta)
        self.beta_logit = _bits(p.beta) if fused_beta else None
        self.a_log = _f32(getattr(p, "a_log", None))
        self.dt_bias = _f32(getattr(p, "dt_bias", None))
        st = p.state if initial_state is None else initial_state
        self.s0 = _f32(st) if use_initial_state else None
        self.N = len(self.cu) - 1
        self.HK = int(p.k.shape[1])
        self.HV = int(p.v.shape[1])
        self.K = int(p.k.shape[2])
        self.V = int(p.v.shape[2])
        self.scale = float(self.K ** -0.5 if scale is None or scale <= 0 else scale)
        self.l2norm = bool(p.l2norm)
        self.nh = int(getattr(p, "num_householder", 1) or 1)
        self._st = _Problem(self.N, self.HK, self.HV, self.K, self.V, int(self.l2norm), self.scale,
                            _ptr(self.cu), _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.g),
                            _ptr(self.beta), _ptr(self.s0), _ptr(self.beta_logit), _ptr(self.a_log),
                            _ptr(self.dt_bias), 0, None, None, self.nh)

    def lengths(self) -> List[int]:
        return [int(self.cu[i + 1] - self.cu[i]) for i in range(self.N)]

    def all_units(self) -> List[Tuple[int, int]]:
        return [(n, h) for n in range(self.N) for h in range(self.HV)]

    def run_units(self, units: Sequence[Tuple[int, int]], want_o: bool = True,
                  want_state: bool = True, want_transition: bool = False,
                  num_threads: Optional[int] = None, checkpoint_every: int = 0) -> Dict[str, list]:
        """Runs the listed (seq, v-head) units; returns per-unit fp64 arrays
        (with checkpoint_every = n > 0 also each unit's state series,
        [ceil(len / n), K, V])."""
        lib = _load()
        units = list(units)
        nu = len(units)
        seq = np.array([u[0] for u in units], dtype=np.int32)
        head = np.array([u[1] for u in units], dtype=np.int32)
        for s, h in units:
            if not (0 <= s < self.N and 0 <= h < self.HV):
                raise ValueError(f"oracle: unit {(s, h)} out of range (N={self.N}, HV={self.HV})")
        lens = np.array([self.cu[s + 1] - self.cu[s] for s in seq], dtype=np.int64)
        if want_o and self.q is None:
            raise ValueError("oracle: outputs need q")
        offs = np.zeros(nu, dtype=np.int64)
        if nu:
            offs[1:] = np.cumsum(lens * self.V)[:-1]
        o = np.empty(int(lens.sum()) * self.V, dtype=np.float64) if want_o else None
        st = np.empty((nu, self.K, self.V), dtype=np.float64) if want_state else None
        tr = np.empty((nu, self.K, self.K), dtype=np.float64) if want_transition else None
        nt = default_threads() if num_threads is None else num_threads
        n_ck = -(-lens // checkpoint_every) if checkpoint_every > 0 else np.zeros(nu, dtype=np.int64)
        ck_offs = np.zeros(nu, dtype=np.int64)
        if nu:
            ck_offs[1:] = np.cumsum(n_ck * self.K * self.V)[:-1]
        ck = np.empty(max(1, int(n_ck.sum()) * self.K * self.V), dtype=np.float64)
        self._st.checkpoint_every = int(checkpoint_every)
        self._st.checkpoints = _ptr(ck) if checkpoint_every > 0 else None
        self._st.checkpoint_offset = _ptr(ck_offs) if checkpoint_every > 0 else None
        rc = lib.gdn_oracle_run(ctypes.byref(self._st), nu, _ptr(seq), _ptr(head),
                                _ptr(offs) if want_o else None, _ptr(o), _ptr(st), _ptr(tr), nt)
        if rc != 0:
            raise RuntimeError(f"gdn_oracle_run failed with {rc}")
        out: Dict[str, list] = {"units": units}
        if want_o:
            out["o"] = [o[offs[i]:offs[i] + lens[i] * self.V].reshape(int(lens[i]), self.V)
                        for i in range(nu)]
        if want_state:
            out["state"] = [st[i] for i in range(nu)]
        if want_transition:
            out["transition"] = [tr[i] for i in range(nu)]
        if checkpoint_every > 0:
            out["checkpoints"] = [ck[ck_offs[i]:ck_offs[i] + n_ck[i] * self.K * self.V].reshape(
                int(n_ck[i]), self.K, self.V) for i in range(nu)]
        return out

    def run_all(self, want_o: bool = True, want_state: bool = True,
                want_transition: bool = False, num_threads: Optional[int] = None,
                checkpoint_every: int = 0) -> Dict[str, np.ndarray]:
        """Every unit, assembled: o [T, HV, V], state [N, HV, K, V], transition [N, HV, K, K],
        and with checkpoint_every = n > 0 the state series [E, HV, K, V]: sequences in batch
        order, ceil(len / n) entries each, entry j the state after j n tokens."""
        units = self.all_units()
        # longest sequences first so the dynamic schedule balances
        units.sort(key=lambda u: -(self.cu[u[0] + 1] - self.cu[u[0]]))
        res = self.run_units(units, want_o, want_state, want_transition, num_threads, checkpoint_every)
        out: Dict[str, np.ndarray] = {}
        T = int(self.cu[-1]) if self.N else 0
        if want_o:
            o = np.zeros((T, self.HV, self.V), dtype=np.float64)
            for (n, h), arr in zip(units, res["o"]):
                o[self.cu[n]:self.cu[n + 1], h, :] = arr
            out["o"] = o
        if want_state:
            s = np.zeros((self.N, self.HV, self.K, self.V), dtype=np.float64)
            for (n, h), arr in zip(units, res["state"]):
                s[n, h] = arr
            out["state"] = s
        if want_transition:
            t = np.zeros((self.N, self.HV, self.K, self.K), dtype=np.float64)
            for (n, h), arr in zip(units, res["transition"]):
                t[n, h] = arr
            out["transition"] = t
        if checkpoint_every > 0:
            n_ck = [-(-l // checkpoint_every) for l in self.lengths()]
            base = np.concatenate([[0], np.cumsum(n_ck)]).astype(np.int64)
            c = np.zeros((int(base[-1]), self.HV, self.K, self.V), dtype=np.float64)
            for (n, h), arr in zip(units, res["checkpoints"]):
                c[base[n]:base[n + 1], h] = arr
            out["checkpoints"] = c
        return out


def backward(problem, d_o=None, d_final=None, scale: Optional[float] = None,
             num_threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Gradients of the forward (plain inputs: fp32 beta, natural-log gate, n = 1) for
    upstream gradients d_o [T, HV, V] and d_final [N, HV, K, V] (None: zeros): dq, dk
    [T, HK, K] (summed over the value heads of each q/k head), dv [T, HV, V], dg, dbeta
    [T, HV] and d_init [N, HV, K, V], all fp64 (see gdn_oracle.c)."""
    o = Oracle(problem, scale=scale)
    if o.beta_logit is not None or o.a_log is not None or o.nh != 1:
        raise ValueError("oracle backward: plain inputs only")
    lib = _load()
    N, HK, HV, K, V = o.N, o.HK, o.HV, o.K, o.V
    T = int(o.cu[-1]) if N else 0
    units = o.all_units()
    lens = np.array([o.cu[n + 1] - o.cu[n] for n, _ in units], dtype=np.int64)
    offs = np.zeros(len(units), dtype=np.int64)
    if units:
        offs[1:] = np.cumsum(lens)[:-1]
    rows = int(lens.sum())
    seq = np.array([u[0] for u in units], dtype=np.int32)
    head = np.array([u[1] for u in units], dtype=np.int32)
    dop = None
    if d_o is not None:
        d_o = np.asarray(d_o, dtype=np.float64)
        dop = np.ascontiguousarray(np.concatenate(
            [d_o[o.cu[n]:o.cu[n + 1], h, :] for n, h in units], axis=0) if units else np.zeros((0, V)))
    dfp = None
    if d_final is not None:
        d_final = np.asarray(d_final, dtype=np.float64)
        dfp = np.ascontiguousarray(np.stack([d_final[n, h] for n, h in units]) if units else np.zeros((0, K, V)))
    dq = np.zeros((max(rows, 1), K))
    dk = np.zeros((max(rows, 1), K))
    dv = np.zeros((max(rows, 1), V))
    dg = np.zeros(max(rows, 1))
    db = np.zeros(max(rows, 1))
    di = np.zeros((max(len(units), 1), K, V))
    nt = default_threads() if num_threads is None else num_threads
    rc = lib.gdn_oracle_backward(ctypes.byref(o._st), len(units), _ptr(seq), _ptr(head), _ptr(offs), _ptr(dop),
                                 _ptr(dfp), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(di), nt)
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_backward failed with {rc}")
    out = {"dq": np.zeros((T, HK, K)), "dk": np.zeros((T, HK, K)), "dv": np.zeros((T, HV, V)),
           "dg": np.zeros((T, HV)), "dbeta": np.zeros((T, HV)), "d_init": np.zeros((N, HV, K, V))}
    G = HV // HK
    for i, (n, h) in enumerate(units):
        a, b = o.cu[n], o.cu[n + 1]
        r = slice(offs[i], offs[i] + lens[i])
        out["dq"][a:b, h // G] += dq[r]
        out["dk"][a:b, h // G] += dk[r]
        out["dv"][a:b, h] = dv[r]
        out["dg"][a:b, h] = dg[r]
        out["dbeta"][a:b, h] = db[r]
        out["d_init"][n, h] = di[i]
    return out


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 in fp64 (0 when both are zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((x - ref).ravel()))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
