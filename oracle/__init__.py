"""fp64 CPU oracle for the KDA state recurrence -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and
shares no code with it: the arithmetic lives in ``kda_oracle.c`` (plain C,
IEEE double, libm ``exp``), written from the definitions on the pages:

* "Kimi K3: Bounded Decay and Delta Memory", section "Formula and
  conventions": the bounded gate g = g_min * sigmoid(e^A z), alpha = e^g,
  and the fade / correct / read recurrence; its contract table fixes the
  shapes, the empty-sequence rule and the absence of a query scale.
* "KDARecurrent", section "The state recurrence in source order": the same
  loop order.

This module only marshals numpy arrays (converted to float64, contiguous)
into the C functions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")


def compile_oracle(src: str, out: str) -> str:
    """gcc -O2 -fopenmp: the oracle as written, no fast-math."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile the C oracle next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_oracle(_SRC, _LIB)
    return _LIB


def _open(path):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.kda_oracle_bounded_decay.argtypes = [dp, dp, dp, ctypes.c_double, i64, i64, i64, ctypes.c_int, dp]
    lib.kda_oracle_bounded_decay.restype = None
    lib.kda_oracle_scan.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.POINTER(i64), i64,
                                    i64, i64, i64, i64, i64, ctypes.c_double, dp, dp, ctypes.c_int]
    lib.kda_oracle_scan.restype = ctypes.c_int
    lib.kda_oracle_bounded_decay_bwd.argtypes = [dp, dp, dp, ctypes.c_double, i64, i64, i64, dp, ctypes.c_int,
                                                 dp, dp, dp]
    lib.kda_oracle_bounded_decay_bwd.restype = None
    lib.kda_oracle_scan_bwd.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.POINTER(i64), i64, i64, i64, i64, i64, i64,
                                        ctypes.c_double, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.kda_oracle_scan_bwd.restype = ctypes.c_int
    lib.kda_oracle_max_threads.argtypes = []
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """Handle on one compiled copy of the C oracle."""

    def __init__(self, path: str = None):
        if path is None:
            path = build()
        self.path = path
        self._lib = _open(path)

    def max_threads(self) -> int:
        return int(self._lib.kda_oracle_max_threads())


    def bounded_decay(self, z, log_scale, g_min: float = -5.0, bias=None, out_log: bool = False) -> np.ndarray:
        """alpha = exp(g_min * sigmoid(e^{log_scale[h]} (z + bias[h, c]))) in float64.

        z: [..., H, K]; log_scale: [H]; bias: [H, K] / [H*K] or None.  With
        ``out_log`` the log-decay g is returned instead of alpha.
        """
        z = _f64(z)
        if z.ndim < 2:
            raise ValueError("z must be [..., H, K]")
        H, K = z.shape[-2], z.shape[-1]
        rows = int(np.prod(z.shape[:-2])) if z.ndim > 2 else 1
        ls = _f64(log_scale).reshape(-1)
        if ls.shape[0] != H:
            raise ValueError("log_scale must have H entries")
        b = None if bias is None else _f64(bias).reshape(-1)
        if b is not None and b.shape[0] != H * K:
            raise ValueError("bias must have H*K entries")
        out = np.empty_like(z)
        self._lib.kda_oracle_bounded_decay(_ptr(z), _ptr(ls), _ptr(b), float(g_min), rows, H, K,
                                         1 if out_log else 0, _ptr(out))
        return out


    def scan(self, q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, scale: float = 1.0,
             nthreads: int = 0):
        """Token-by-token KDA scan in float64.  Returns (out [B,T,H,V], final_state [N,H,K,V]).

        q, k: [B,T,H,K]; v: [B,T,H,V]; alpha: [B,T,H,K] retention; beta: [B,T,H];
        initial_state: [N,H,K,V] or None (zeros); cu_seqlens: int [N+1] offsets into
        the single batch row (B must be 1) or None (N = B).
        """
        q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
        if q.ndim != 4 or v.ndim != 4:
            raise ValueError("q, k, v must be 4-D")
        B, T, H, K = q.shape
        V = v.shape[3]
        if k.shape != q.shape or alpha.shape != q.shape or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
            raise ValueError("inconsistent shapes")
        cu = None
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).reshape(-1))
            N = cu.shape[0] - 1
        else:
            N = B
        s0 = None if initial_state is None else _f64(initial_state)
        if s0 is not None and s0.shape != (N, H, K, V):
            raise ValueError("initial_state must be [N,H,K,V]")
        out = np.zeros((B, T, H, V), dtype=np.float64)
        fin = np.zeros((N, H, K, V), dtype=np.float64)
        rc = self._lib.kda_oracle_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0),
                                     None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     N, B, T, H, K, V, float(scale), _ptr(out), _ptr(fin), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (cu_seqlens inconsistent with B/T?)")
        return out, fin


    def bounded_decay_bwd(self, z, log_scale, grad, g_min: float = -5.0, bias=None, grad_is_log: bool = False):
        """Gradients of bounded_decay: returns (dz [..., H, K], dlog_scale [H], dbias [H, K]).

        grad is dL/dalpha, or dL/dg with ``grad_is_log``; dbias is returned whether or not a
        bias is given (the gradient a featurewise bias would receive).
        """
        z = _f64(z)
        H, K = z.shape[-2], z.shape[-1]
        rows = int(np.prod(z.shape[:-2])) if z.ndim > 2 else 1
        ls = _f64(log_scale).reshape(-1)
        gr = _f64(grad)
        if gr.shape != z.shape or ls.shape[0] != H:
            raise ValueError("grad must match z and log_scale must have H entries")
        b = None if bias is None else _f64(bias).reshape(-1)
        dz = np.empty_like(z)
        dls = np.empty(H)
        db = np.empty(H * K)
        self._lib.kda_oracle_bounded_decay_bwd(_ptr(z), _ptr(ls), _ptr(b), float(g_min), rows, H, K, _ptr(gr),
                                             1 if grad_is_log else 0, _ptr(dz), _ptr(dls), _ptr(db))
        return dz, dls, db.reshape(H, K)

    def scan_bwd(self, q, k, v, alpha, beta, d_out, initial_state=None, d_final_state=None, cu_seqlens=None,
                 scale: float = 1.0, nthreads: int = 0):
        """Gradients of scan for L = <d_out, out> + <d_final_state, final_state>.

        Returns (dq, dk, dv, dalpha, dbeta, d_initial_state) in float64, shaped like
        q, k, v, alpha, beta and [N, H, K, V].  d_final_state None means zeros.
        """
        q, k, v, alpha, beta, d_out = (_f64(x) for x in (q, k, v, alpha, beta, d_out))
        B, T, H, K = q.shape
        V = v.shape[3]
        if k.shape != q.shape or alpha.shape != q.shape or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H) \
                or d_out.shape != v.shape:
            raise ValueError("inconsistent shapes")
        cu = None
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).reshape(-1))
            N = cu.shape[0] - 1
        else:
            N = B
        s0 = None if initial_state is None else _f64(initial_state)
        dsT = None if d_final_state is None else _f64(d_final_state)
        for x in (s0, dsT):
            if x is not None and x.shape != (N, H, K, V):
                raise ValueError("states must be [N,H,K,V]")
        dq, dk, da = (np.zeros_like(q) for _ in range(3))
        dv = np.zeros_like(v)
        db = np.zeros_like(beta)
        ds0 = np.zeros((N, H, K, V))
        rc = self._lib.kda_oracle_scan_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0),
                                         None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         N, B, T, H, K, V, float(scale), _ptr(d_out), _ptr(dsT), _ptr(dq), _ptr(dk),
                                         _ptr(dv), _ptr(da), _ptr(db), _ptr(ds0), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (cu_seqlens inconsistent with B/T?)")
        return dq, dk, dv, da, db, ds0


_default = None


def _get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def max_threads() -> int:
    return _get().max_threads()


def bounded_decay(*a, **kw):
    return _get().bounded_decay(*a, **kw)


def scan(*a, **kw):
    return _get().scan(*a, **kw)


def scan_bwd(*a, **kw):
    return _get().scan_bwd(*a, **kw)


def bounded_decay_bwd(*a, **kw):
    return _get().bounded_decay_bwd(*a, **kw)
