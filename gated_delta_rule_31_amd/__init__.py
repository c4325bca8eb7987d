"""MI355X (gfx950) Kimi Delta Attention (KDA) state recurrence.

A thin Python binding over the C ABI of ``include/kda.h`` (``libkda.so``, built
in-tree by ``gated_delta_rule_31_amd/build.py``).  PyTorch supplies device memory
and the current stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing, or the tensors are not
on a GPU, these functions raise.

Entry points (same names as the C ABI, minus the ``kda_`` prefix where noted):

* ``bounded_decay(logits, log_scale, lower_bound=-5, bias=None, out_log=False)``
  -- the K3 gate alpha = exp(g_min * sigmoid(e^A (z + bias))) (or g itself).
* ``chunk_fwd(q, k, v, gate, beta, ...)`` -- chunkwise prefill with optional
  initial / final state and packed sequences (``cu_seqlens``).  By default
  (``TWO_PASS``) it runs in its two-kernel form over a workspace (a pre-pass over all
  chunks, then the serial part); ``two_pass=False`` selects the single kernel, and
  ``workspace=`` passes a caller-owned buffer of ``chunk_fwd_workspace_size(...)``
  bytes.
* ``recurrent_step(q, k, v, gate, beta, state, ...)`` -- one decode token, state
  updated in place.
* ``recurrent_fwd(q, k, v, gate, beta, ...)`` -- the prefill contract of ``chunk_fwd``
  evaluated token by token (short sequences; no chunk size, any alpha in [0, 1]).
* ``chunk_fwd_fused_gate`` / ``recurrent_fwd_fused_gate`` / ``recurrent_step_fused_gate``
  -- the same calls with
  the gate applied inside the kernel from its logits (``log_scale``, ``bias``,
  ``lower_bound``), so no float32 gate tensor is made.
* ``chunk_bwd(q, k, v, gate, beta, d_out, ...)`` -- gradients of ``chunk_fwd`` into q, k,
  v, the gate, beta and the initial state; ``bounded_decay_bwd`` -- gradients of the gate
  into its logits, log-scale and bias.
* ``recurrent_kda(q, k, v, alpha, beta, initial_state=None)`` -- the functional
  (output, final_state) form of the pages' operator contract, on ``chunk_fwd``; it is
  differentiable (autograd through ``chunk_bwd``), and so is ``bounded_decay`` when its
  inputs require grad (through ``bounded_decay_bwd``).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["bounded_decay", "chunk_fwd", "recurrent_step", "recurrent_kda", "KDAError", "chunk_fwd_supported",
           "chunk_fwd_fused_gate", "recurrent_step_fused_gate", "recurrent_fwd", "recurrent_fwd_fused_gate",
           "library_path", "abi_version", "GATE_ALPHA", "GATE_LOG", "chunk_bwd", "chunk_bwd_workspace_size",
           "bounded_decay_bwd", "chunk_fwd_workspace_size", "TWO_PASS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
GATE_ALPHA, GATE_LOG = 0, 1
QK_L2NORM, BETA_LOGITS, STATE_VK = 1, 2, 4  # input-preparation flags of the fused-gate calls


def _flags(qk_l2norm: bool, beta_logits: bool, state_vk: bool) -> int:
    return (QK_L2NORM if qk_l2norm else 0) | (BETA_LOGITS if beta_logits else 0) | (STATE_VK if state_vk else 0)
_STATUS = {0: "ok", 1: "null pointer", 2: "bad shape", 3: "bad dtype", 4: "unsupported",
           5: "bad argument", 6: "alias", 7: "hip error"}


class KDAError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__("%s failed: %s (status %d)%s" % (fn, _STATUS.get(status, "?"), status,
                                                         (": " + detail) if detail else ""))


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libkda.so is not built (%s); run gated_delta_rule_31_amd/build.py" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_uint
    lib.kda_bounded_decay.argtypes = [vp, i32, vp, vp, f32, i64, i32, i32, i32, vp, vp]
    lib.kda_bounded_decay.restype = i32
    sz = ctypes.c_size_t
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, i64, i32, i32,
                                  i32, i32, f32, vp, i32, vp, sz, vp]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_recurrent_step.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, f32, vp,
                                       i32, vp]
    lib.kda_recurrent_step.restype = i32
    lib.kda_chunk_fwd_fused_gate.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, u32, vp, vp, vp, vp, i32, i32,
                                             i64, i32, i32, i32, i32, f32, vp, i32, vp, sz, vp]
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, i32]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd_fused_gate.restype = i32
    lib.kda_chunk_fwd_fused_gate_noalloc.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, u32, vp, vp, vp, vp, i32, i32,
                                                     i64, i32, i32, i32, i32, f32, vp, i32, vp]
    lib.kda_chunk_fwd_fused_gate_noalloc.restype = i32
    lib.kda_noalloc_scratch_bytes.argtypes = []
    lib.kda_noalloc_scratch_bytes.restype = sz
    lib.kda_recurrent_step_fused_gate.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, u32, vp, vp, i32, i32, i32,
                                                  i32, f32, vp, i32, vp]
    lib.kda_recurrent_step_fused_gate.restype = i32
    lib.kda_recurrent_fwd.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32,
                                      f32, vp, i32, vp]
    lib.kda_recurrent_fwd.restype = i32
    lib.kda_recurrent_fwd_fused_gate.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, u32, vp, vp, vp, vp, i32, i32,
                                                 i64, i32, i32, i32, f32, vp, i32, vp]
    lib.kda_recurrent_fwd_fused_gate.restype = i32
    lib.kda_chunk_bwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    lib.kda_chunk_bwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_bwd.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, vp, i32,
                                  vp, vp, vp, vp, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.kda_chunk_bwd.restype = i32
    lib.kda_bounded_decay_bwd.argtypes = [vp, i32, vp, vp, f32, i64, i32, i32, vp, i32, vp, i32, vp, vp, vp]
    lib.kda_bounded_decay_bwd.restype = i32
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = i32
    lib.kda_chunk_fwd_supported.argtypes = [i32, i32, i32, i32]
    lib.kda_chunk_fwd_supported.restype = i32
    lib.kda_last_hip_error.argtypes = []
    lib.kda_last_hip_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def abi_version() -> int:
    return int(_load().kda_abi_version())


def chunk_fwd_supported(dtype: torch.dtype, K: int, V: int, chunk_size: int) -> int:
    """Value columns per workgroup kda_chunk_fwd uses for this shape, 0 if unsupported."""
    return int(_load().kda_chunk_fwd_supported(_dtype_code(dtype), int(K), int(V), int(chunk_size)))


# Default of the ``two_pass`` argument of the chunk prefill calls: with True (and a shape
# the two-kernel form supports) a workspace is taken from torch's allocator and the
# pre-pass + chain kernels run; with False the single chunk kernel runs.
TWO_PASS = True


def chunk_fwd_workspace_size(dtype: torch.dtype, B: int, T: int, H: int, K: int, V: int, chunk_size: int = 32,
                             num_seqs: int = 0, varlen: bool = False) -> int:
    """Bytes of workspace the two-kernel prefill needs (0: that form does not support the shape)."""
    return int(_load().kda_chunk_fwd_workspace_size(_dtype_code(dtype), int(B), int(T), int(num_seqs),
                                                    1 if varlen else 0, int(H), int(K), int(V), int(chunk_size)))


def _chunk_workspace(two_pass, workspace, q, N, V, chunk_size, varlen):
    """The (pointer, bytes) workspace arguments of a chunk prefill call."""
    if workspace is not None:
        if workspace.device != q.device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the device of q")
        return workspace, workspace.numel()
    explicit = two_pass is not None
    if not (two_pass if explicit else TWO_PASS):
        return None, 0
    B, T, H, K = q.shape
    n = chunk_fwd_workspace_size(q.dtype, B, T, H, K, V, chunk_size, N, varlen)
    if n == 0:
        if explicit:  # asked for by name: no silent switch to the single kernel
            raise KDAError("kda_chunk_fwd_workspace_size", 4, "the two-kernel form does not support this shape")
        return None, 0
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    return ws, n


def _check(fn: str, status: int):
    if status != 0:
        detail = _load().kda_last_hip_error().decode() if status == 7 else ""
        if status in (2, 3, 4, 5, 6):
            raise ValueError(str(KDAError(fn, status, detail)))
        raise KDAError(fn, status, detail)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise ValueError("unsupported dtype %s (float32 or bfloat16)" % t)


def _dev(x: Optional[torch.Tensor], name: str, dtype=None) -> Optional[torch.Tensor]:
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.device.type != "cuda":
        raise ValueError("%s must be on the GPU (got %s)" % (name, x.device))
    if x.requires_grad and torch.is_grad_enabled():
        raise ValueError("%s requires grad: the raw kernels do not record autograd; use recurrent_kda / "
                         "bounded_decay, or call chunk_bwd yourself" % name)
    if dtype is not None and x.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, x.dtype))
    return x.contiguous()


def _ptr(x: Optional[torch.Tensor]):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(x: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)


def _needs_grad(*xs) -> bool:
    return torch.is_grad_enabled() and any(isinstance(x, torch.Tensor) and x.requires_grad for x in xs)


def bounded_decay(logits: torch.Tensor, log_scale: torch.Tensor, lower_bound: float = -5.0,
                  bias: Optional[torch.Tensor] = None, out_log: bool = False,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Retention factors alpha [..., H, K] (float32) from logits [..., H, K]
    (float32 or bfloat16); with ``out_log`` the log-decay g instead.  Differentiable in
    logits, log_scale and bias when any of them requires grad (``out`` is then not
    accepted)."""
    if _needs_grad(logits, log_scale, bias):
        if out is not None:
            raise ValueError("out= is not supported when gradients are recorded")
        return _BoundedDecayFn.apply(logits, log_scale, bias, float(lower_bound), bool(out_log))
    logits = _dev(logits, "logits")
    log_scale = _dev(log_scale, "log_scale", torch.float32)
    bias = _dev(bias, "bias", torch.float32)
    if logits.dim() < 2:
        raise ValueError("logits must be [..., H, K]")
    H, K = logits.shape[-2], logits.shape[-1]
    if log_scale.numel() != H or (bias is not None and bias.numel() != H * K):
        raise ValueError("log_scale must be [H] and bias [H, K]")
    rows = logits.numel() // (H * K) if H * K else 0
    if out is None:
        out = torch.empty(logits.shape, dtype=torch.float32, device=logits.device)
    elif out.shape != logits.shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like logits")
    with torch.cuda.device(logits.device):
        st = _load().kda_bounded_decay(_ptr(logits), _dtype_code(logits.dtype), _ptr(log_scale),
                                       _ptr(bias), float(lower_bound), rows, H, K,
                                       GATE_LOG if out_log else GATE_ALPHA, _ptr(out), _stream(logits))
    _check("kda_bounded_decay", st)
    return out


def _chunk_common(q, k, v, beta, initial_state, output_final_state, cu_seqlens, out_dtype, out, final_state,
                  state_vk: bool = False):
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    beta = _dev(beta, "beta", torch.float32)
    initial_state = _dev(initial_state, "initial_state", torch.float32)
    cu_seqlens = _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, D]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes: q %s k %s v %s beta %s" % (
            tuple(q.shape), tuple(k.shape), tuple(v.shape), tuple(beta.shape)))
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    sshape = (N, H, V, K) if state_vk else (N, H, K, V)
    if initial_state is not None and initial_state.shape != sshape:
        raise ValueError("initial_state must be %s" % (list(sshape),))
    od = out_dtype or v.dtype
    if out is None:
        out = torch.empty((B, T, H, V), dtype=od, device=q.device)
    elif out.shape != (B, T, H, V) or out.dtype != od or not out.is_contiguous():
        raise ValueError("out must be contiguous [B,T,H,V] of the output dtype")
    if output_final_state and final_state is None:
        final_state = torch.empty(sshape, dtype=torch.float32, device=q.device)
    if final_state is not None and (final_state.shape != sshape or final_state.dtype != torch.float32
                                    or not final_state.is_contiguous()):
        raise ValueError("final_state must be contiguous float32 %s" % (list(sshape),))
    return q, k, v, beta, initial_state, cu_seqlens, N, od, out, final_state


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor,
              beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              output_final_state: bool = True, cu_seqlens: Optional[torch.Tensor] = None,
              chunk_size: int = 32, scale: float = 1.0, gate_is_log: bool = False,
              out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None, two_pass: Optional[bool] = None,
              workspace: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise prefill.  q, k [B,T,H,K]; v [B,T,H,V] (one dtype, float32 or
    bfloat16); gate [B,T,H,K] float32 (alpha, or ln alpha with ``gate_is_log``);
    beta [B,T,H] float32; initial_state [N,H,K,V] float32 or None; cu_seqlens
    int32 [N+1] (B == 1) or None.  Returns (out [B,T,H,V], final_state [N,H,K,V]
    or None).  ``final_state`` may be passed in (it may be ``initial_state``).
    ``two_pass`` (default ``TWO_PASS``): pre-pass + chain kernels over a workspace
    (``workspace``, uint8, or one from torch's allocator) instead of the single kernel."""
    q, k, v, beta, initial_state, cu_seqlens, N, od, out, final_state = _chunk_common(
        q, k, v, beta, initial_state, output_final_state, cu_seqlens, out_dtype, out, final_state)
    gate = _dev(gate, "gate", torch.float32)
    if gate.shape != q.shape:
        raise ValueError("gate must be shaped like q")
    B, T, H, K = q.shape
    V = v.shape[-1]
    ws, nws = _chunk_workspace(two_pass, workspace, q, N, V, chunk_size, cu_seqlens is not None)
    with torch.cuda.device(q.device):
        st = _load().kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(gate),
                                   GATE_LOG if gate_is_log else GATE_ALPHA, _ptr(beta),
                                   _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N, B, T,
                                   H, K, V, int(chunk_size), float(scale), _ptr(out), _dtype_code(od),
                                   _ptr(ws), nws, _stream(q))
    _check("kda_chunk_fwd", st)
    return out, final_state


def _gate_params(logits, log_scale, bias, like: torch.Tensor):
    logits = _dev(logits, "logits", like.dtype)
    log_scale = _dev(log_scale, "log_scale", torch.float32)
    bias = _dev(bias, "bias", torch.float32)
    H, K = like.shape[-2], like.shape[-1]
    if logits.shape != like.shape:
        raise ValueError("logits must be shaped like q")
    if log_scale.numel() != H or (bias is not None and bias.numel() != H * K):
        raise ValueError("log_scale must be [H] and bias [H, K]")
    return logits, log_scale, bias


def chunk_fwd_fused_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, logits: torch.Tensor,
                         log_scale: torch.Tensor, beta: torch.Tensor, bias: Optional[torch.Tensor] = None,
                         lower_bound: float = -5.0, initial_state: Optional[torch.Tensor] = None,
                         output_final_state: bool = True, cu_seqlens: Optional[torch.Tensor] = None,
                         chunk_size: int = 32, scale: float = 1.0, out_dtype: Optional[torch.dtype] = None,
                         out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                         qk_l2norm: bool = False, beta_logits: bool = False, state_vk: bool = False,
                         two_pass: Optional[bool] = None, workspace: Optional[torch.Tensor] = None
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd`` with alpha = exp(lower_bound * sigmoid(e^log_scale (logits + bias)))
    computed inside the kernel.  logits [B,T,H,K] in the dtype of q; log_scale [H] and
    bias [H,K] float32; lower_bound in [-5, 0).  ``qk_l2norm``: q and k are normalised
    over K in the kernel; ``beta_logits``: beta holds logits (sigmoid in the kernel);
    ``state_vk``: states are [N,H,V,K]; ``two_pass``, ``workspace``: as in ``chunk_fwd``."""
    q, k, v, beta, initial_state, cu_seqlens, N, od, out, final_state = _chunk_common(
        q, k, v, beta, initial_state, output_final_state, cu_seqlens, out_dtype, out, final_state, state_vk)
    logits, log_scale, bias = _gate_params(logits, log_scale, bias, q)
    B, T, H, K = q.shape
    V = v.shape[-1]
    ws, nws = _chunk_workspace(two_pass, workspace, q, N, V, chunk_size, cu_seqlens is not None)
    with torch.cuda.device(q.device):
        st = _load().kda_chunk_fwd_fused_gate(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(logits),
                                              _ptr(log_scale), _ptr(bias), float(lower_bound),
                                              _flags(qk_l2norm, beta_logits, state_vk), _ptr(beta),
                                              _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N, B,
                                              T, H, K, V, int(chunk_size), float(scale), _ptr(out),
                                              _dtype_code(od), _ptr(ws), nws, _stream(q))
    _check("kda_chunk_fwd_fused_gate", st)
    return out, final_state


def noalloc_scratch_bytes() -> int:
    """Bytes of the library's fixed per-device workspace used by the ``*_noalloc`` call."""
    return int(_load().kda_noalloc_scratch_bytes())


def chunk_fwd_fused_gate_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, logits: torch.Tensor,
                                 log_scale: torch.Tensor, beta: torch.Tensor, out: torch.Tensor,
                                 bias: Optional[torch.Tensor] = None, lower_bound: float = -5.0,
                                 initial_state: Optional[torch.Tensor] = None,
                                 final_state: Optional[torch.Tensor] = None,
                                 cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 32,
                                 scale: float = 1.0, qk_l2norm: bool = False, beta_logits: bool = False,
                                 state_vk: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd_fused_gate`` in its two-kernel form with its workspace in the library's
    fixed per-device array (``noalloc_scratch_bytes()``): nothing is allocated, by the
    library or here -- ``out`` (and ``final_state`` if wanted) come from the caller.  Shapes
    whose workspace exceeds the array raise ValueError (unsupported).  Calls that overlap
    on one GPU race on the array."""
    q, k, v, beta, initial_state, cu_seqlens, N, od, out, final_state = _chunk_common(
        q, k, v, beta, initial_state, False, cu_seqlens, out.dtype, out, final_state, state_vk)
    logits, log_scale, bias = _gate_params(logits, log_scale, bias, q)
    B, T, H, K = q.shape
    V = v.shape[-1]
    with torch.cuda.device(q.device):
        st = _load().kda_chunk_fwd_fused_gate_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype),
                                                      _ptr(logits), _ptr(log_scale), _ptr(bias), float(lower_bound),
                                                      _flags(qk_l2norm, beta_logits, state_vk), _ptr(beta),
                                                      _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N,
                                                      B, T, H, K, V, int(chunk_size), float(scale), _ptr(out),
                                                      _dtype_code(od), _stream(q))
    _check("kda_chunk_fwd_fused_gate_noalloc", st)
    return out, final_state


def recurrent_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor,
                  beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                  output_final_state: bool = True, cu_seqlens: Optional[torch.Tensor] = None,
                  scale: float = 1.0, gate_is_log: bool = False, out_dtype: Optional[torch.dtype] = None,
                  out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd``'s contract evaluated token by token (for short sequences); no chunk
    size and no bound on the log-decay."""
    q, k, v, beta, initial_state, cu_seqlens, N, od, out, final_state = _chunk_common(
        q, k, v, beta, initial_state, output_final_state, cu_seqlens, out_dtype, out, final_state)
    gate = _dev(gate, "gate", torch.float32)
    if gate.shape != q.shape:
        raise ValueError("gate must be shaped like q")
    B, T, H, K = q.shape
    V = v.shape[-1]
    with torch.cuda.device(q.device):
        st = _load().kda_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(gate),
                                       GATE_LOG if gate_is_log else GATE_ALPHA, _ptr(beta), _ptr(initial_state),
                                       _ptr(final_state), _ptr(cu_seqlens), N, B, T, H, K, V, float(scale),
                                       _ptr(out), _dtype_code(od), _stream(q))
    _check("kda_recurrent_fwd", st)
    return out, final_state


def recurrent_fwd_fused_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, logits: torch.Tensor,
                             log_scale: torch.Tensor, beta: torch.Tensor, bias: Optional[torch.Tensor] = None,
                             lower_bound: float = -5.0, initial_state: Optional[torch.Tensor] = None,
                             output_final_state: bool = True, cu_seqlens: Optional[torch.Tensor] = None,
                             scale: float = 1.0, out_dtype: Optional[torch.dtype] = None,
                             out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                             qk_l2norm: bool = False, beta_logits: bool = False, state_vk: bool = False
                             ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``recurrent_fwd`` with the gate evaluated inside the kernel from its logits (and
    the input-preparation options of ``chunk_fwd_fused_gate``)."""
    q, k, v, beta, initial_state, cu_seqlens, N, od, out, final_state = _chunk_common(
        q, k, v, beta, initial_state, output_final_state, cu_seqlens, out_dtype, out, final_state, state_vk)
    logits, log_scale, bias = _gate_params(logits, log_scale, bias, q)
    B, T, H, K = q.shape
    V = v.shape[-1]
    with torch.cuda.device(q.device):
        st = _load().kda_recurrent_fwd_fused_gate(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(logits),
                                                  _ptr(log_scale), _ptr(bias), float(lower_bound),
                                                  _flags(qk_l2norm, beta_logits, state_vk), _ptr(beta),
                                                  _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N, B,
                                                  T, H, K, V, float(scale), _ptr(out), _dtype_code(od),
                                                  _stream(q))
    _check("kda_recurrent_fwd_fused_gate", st)
    return out, final_state


def _step_common(q, k, v, beta, state, out_dtype, out, state_vk: bool = False):
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    beta = _dev(beta, "beta", torch.float32)
    if not isinstance(state, torch.Tensor) or state.device.type != "cuda" or state.dtype != torch.float32 \
            or not state.is_contiguous():
        raise ValueError("state must be a contiguous float32 GPU tensor (it is updated in place)")
    if q.dim() != 3:
        raise ValueError("q must be [B, H, K]")
    B, H, K = q.shape
    V = v.shape[-1]
    sshape = (B, H, V, K) if state_vk else (B, H, K, V)
    if k.shape != q.shape or v.shape != (B, H, V) or beta.shape != (B, H) or state.shape != sshape:
        raise ValueError("inconsistent shapes")
    od = out_dtype or v.dtype
    if out is None:
        out = torch.empty((B, H, V), dtype=od, device=q.device)
    elif out.shape != (B, H, V) or out.dtype != od or not out.is_contiguous():
        raise ValueError("out must be contiguous [B,H,V] of the output dtype")
    return q, k, v, beta, od, out


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor,
                   beta: torch.Tensor, state: torch.Tensor, scale: float = 1.0,
                   gate_is_log: bool = False, out_dtype: Optional[torch.dtype] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode token.  q, k [B,H,K]; v [B,H,V]; gate [B,H,K] float32; beta [B,H]
    float32; state [B,H,K,V] float32 contiguous, updated in place.  Returns out [B,H,V]."""
    q, k, v, beta, od, out = _step_common(q, k, v, beta, state, out_dtype, out)
    gate = _dev(gate, "gate", torch.float32)
    if gate.shape != q.shape:
        raise ValueError("gate must be shaped like q")
    B, H, K = q.shape
    V = v.shape[-1]
    with torch.cuda.device(q.device):
        st = _load().kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(gate),
                                        GATE_LOG if gate_is_log else GATE_ALPHA, _ptr(beta), _ptr(state),
                                        B, H, K, V, float(scale), _ptr(out), _dtype_code(od), _stream(q))
    _check("kda_recurrent_step", st)
    return out


def recurrent_step_fused_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, logits: torch.Tensor,
                              log_scale: torch.Tensor, beta: torch.Tensor, state: torch.Tensor,
                              bias: Optional[torch.Tensor] = None, lower_bound: float = -5.0,
                              scale: float = 1.0, out_dtype: Optional[torch.dtype] = None,
                              out: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                              beta_logits: bool = False, state_vk: bool = False) -> torch.Tensor:
    """``recurrent_step`` with the gate computed inside the kernel from logits [B,H,K]
    (dtype of q), log_scale [H], bias [H,K] or None and lower_bound < 0; the
    input-preparation options of ``chunk_fwd_fused_gate`` (state [B,H,V,K] with
    ``state_vk``)."""
    q, k, v, beta, od, out = _step_common(q, k, v, beta, state, out_dtype, out, state_vk)
    logits, log_scale, bias = _gate_params(logits, log_scale, bias, q)
    B, H, K = q.shape
    V = v.shape[-1]
    with torch.cuda.device(q.device):
        st = _load().kda_recurrent_step_fused_gate(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(logits),
                                                   _ptr(log_scale), _ptr(bias), float(lower_bound),
                                                   _flags(qk_l2norm, beta_logits, state_vk), _ptr(beta),
                                                   _ptr(state), B, H, K, V, float(scale), _ptr(out),
                                                   _dtype_code(od), _stream(q))
    _check("kda_recurrent_step_fused_gate", st)
    return out


def chunk_bwd_workspace_size(B: int, T: int, H: int, K: int, V: int, num_seqs: int = 0,
                             varlen: bool = False) -> int:
    """Bytes of device workspace ``chunk_bwd`` needs for this shape (0: unsupported)."""
    return int(_load().kda_chunk_bwd_workspace_size(int(B), int(T), int(H), int(K), int(V), int(num_seqs),
                                                     1 if varlen else 0))


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor, beta: torch.Tensor,
              d_out: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              d_final_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
              scale: float = 1.0, gate_is_log: bool = False, grad_dtype: Optional[torch.dtype] = None,
              want_d_initial_state: bool = True, workspace: Optional[torch.Tensor] = None):
    """Gradients of ``chunk_fwd`` (same q, k, v, gate, beta, initial_state, cu_seqlens,
    scale) for L = <d_out, out> + <d_final_state, final_state>.  Returns (dq, dk, dv,
    dgate, dbeta, d_initial_state): dq, dk, dv in ``grad_dtype`` (default: the dtype of
    q), dgate float32 (dL/dalpha, or dL/d ln alpha with ``gate_is_log``), dbeta float32,
    d_initial_state [N,H,K,V] float32 or None.  ``workspace``: a uint8 CUDA tensor of at
    least ``chunk_bwd_workspace_size`` bytes, allocated here if not given."""
    q, k, v, beta, initial_state, cu_seqlens, N, _, _, _ = _chunk_common(
        q, k, v, beta, initial_state, False, cu_seqlens, None, None, None)
    gate = _dev(gate, "gate", torch.float32)
    d_out = _dev(d_out, "d_out")
    d_final_state = _dev(d_final_state, "d_final_state", torch.float32)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if gate.shape != q.shape or d_out.shape != v.shape:
        raise ValueError("gate must be shaped like q and d_out like v")
    if d_final_state is not None and d_final_state.shape != (N, H, K, V):
        raise ValueError("d_final_state must be [N,H,K,V]")
    gd = grad_dtype or q.dtype
    dev = q.device
    dq = torch.empty(q.shape, dtype=gd, device=dev)
    dk = torch.empty(q.shape, dtype=gd, device=dev)
    dv = torch.empty(v.shape, dtype=gd, device=dev)
    dgate = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dbeta = torch.empty(beta.shape, dtype=torch.float32, device=dev)
    ds0 = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if want_d_initial_state else None
    need = chunk_bwd_workspace_size(B, T, H, K, V, N, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError("workspace must be a uint8 tensor of at least %d bytes on %s" % (need, dev))
    with torch.cuda.device(dev):
        st = _load().kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(gate),
                                   GATE_LOG if gate_is_log else GATE_ALPHA, _ptr(beta), _ptr(initial_state),
                                   _ptr(cu_seqlens), N, B, T, H, K, V, float(scale), _ptr(d_out),
                                   _dtype_code(d_out.dtype), _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _dtype_code(gd), _ptr(dgate), _ptr(dbeta), _ptr(ds0), _ptr(workspace),
                                   workspace.numel(), _stream(q))
    _check("kda_chunk_bwd", st)
    return dq, dk, dv, dgate, dbeta, ds0


def bounded_decay_bwd(logits: torch.Tensor, log_scale: torch.Tensor, grad: torch.Tensor,
                      lower_bound: float = -5.0, bias: Optional[torch.Tensor] = None, grad_is_log: bool = False,
                      dlogits_dtype: Optional[torch.dtype] = None):
    """Gradients of ``bounded_decay`` given grad = dL/dalpha (or dL/dg with
    ``grad_is_log``).  Returns (d_logits in ``dlogits_dtype`` (default: the logits'
    dtype), d_log_scale [H] float32, d_bias [H, K] float32)."""
    logits = _dev(logits, "logits")
    log_scale = _dev(log_scale, "log_scale", torch.float32)
    bias = _dev(bias, "bias", torch.float32)
    grad = _dev(grad, "grad", torch.float32)
    if logits.dim() < 2 or grad.shape != logits.shape:
        raise ValueError("logits must be [..., H, K] and grad shaped like it")
    H, K = logits.shape[-2], logits.shape[-1]
    if log_scale.numel() != H or (bias is not None and bias.numel() != H * K):
        raise ValueError("log_scale must be [H] and bias [H, K]")
    rows = logits.numel() // (H * K) if H * K else 0
    dd = dlogits_dtype or logits.dtype
    dz = torch.empty(logits.shape, dtype=dd, device=logits.device)
    dls = torch.empty(H, dtype=torch.float32, device=logits.device)
    db = torch.empty((H, K), dtype=torch.float32, device=logits.device)
    with torch.cuda.device(logits.device):
        st = _load().kda_bounded_decay_bwd(_ptr(logits), _dtype_code(logits.dtype), _ptr(log_scale), _ptr(bias),
                                           float(lower_bound), rows, H, K, _ptr(grad),
                                           GATE_LOG if grad_is_log else GATE_ALPHA, _ptr(dz), _dtype_code(dd),
                                           _ptr(dls), _ptr(db), _stream(logits))
    _check("kda_bounded_decay_bwd", st)
    return dz, dls, db


class _BoundedDecayFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, log_scale, bias, lower_bound, out_log):
        with torch.no_grad():
            out = bounded_decay(logits.detach(), log_scale.detach(), lower_bound,
                                None if bias is None else bias.detach(), out_log)
        ctx.save_for_backward(logits, log_scale, bias)
        ctx.lower_bound, ctx.out_log = lower_bound, out_log
        return out

    @staticmethod
    def backward(ctx, grad):
        logits, log_scale, bias = ctx.saved_tensors
        with torch.no_grad():
            dz, dls, db = bounded_decay_bwd(logits.detach(), log_scale.detach(), grad.float().contiguous(),
                                            ctx.lower_bound, None if bias is None else bias.detach(), ctx.out_log)
        return (dz, dls.reshape(log_scale.shape).to(log_scale.dtype),
                None if bias is None else db.reshape(bias.shape).to(bias.dtype), None, None)


class _ChunkKDAFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, alpha, beta, initial_state, chunk_size, scale):
        with torch.no_grad():
            d = lambda x: None if x is None else x.detach()
            out, fin = chunk_fwd(d(q), d(k), d(v), d(alpha), d(beta), initial_state=d(initial_state),
                                 output_final_state=True, chunk_size=chunk_size, scale=scale)
        ctx.save_for_backward(q, k, v, alpha, beta, initial_state)
        ctx.scale = scale
        ctx.has_s0 = initial_state is not None
        return out, fin

    @staticmethod
    def backward(ctx, d_out, d_fin):
        q, k, v, alpha, beta, s0 = ctx.saved_tensors
        if d_out is None:
            d_out = torch.zeros(v.shape, dtype=v.dtype, device=v.device)
        with torch.no_grad():
            d = lambda x: None if x is None else x.detach()
            dq, dk, dv, da, db, ds0 = chunk_bwd(d(q), d(k), d(v), d(alpha), d(beta), d_out.contiguous(),
                                                initial_state=d(s0),
                                                d_final_state=None if d_fin is None else d_fin.float().contiguous(),
                                                scale=ctx.scale, want_d_initial_state=ctx.has_s0)
        return dq, dk, dv, da, db, ds0, None, None


# Smallest retention the chunked prefill accepts: its 16-token rescale factors stay finite
# only while every log-decay is at least -5 (the bounded gate's range, g_min = -5).
CHUNK_MIN_ALPHA = math.exp(-5.0) * (1.0 - 1e-6)


def gate_within_chunk_bound(alpha: torch.Tensor) -> bool:
    """True when every retention factor is at least e^-5, the chunked prefill's
    precondition (one device reduction and a host synchronisation)."""
    return alpha.numel() == 0 or bool(alpha.detach().min() >= CHUNK_MIN_ALPHA)


def recurrent_kda(q, k, v, alpha, beta, initial_state=None, chunk_size: int = 32, scale: float = 1.0,
                  bounded: Optional[bool] = None):
    """PaperLeet ``recurrent_kda`` contract: (output [B,T,H,V], final_state [B,H,K,V]),
    output in the inputs' dtype, every output read after its token's update, inputs
    untouched; T == 0 returns the supplied state (or zeros); any alpha in [0, 1].

    The chunked prefill needs every alpha >= e^-5 (the bounded gate's range); the
    token-recurrent kernel takes any alpha in [0, 1].  ``bounded`` picks the path:
    None checks the smallest alpha on the device (one reduction and a host sync) and
    takes the chunked prefill when the bound holds, the token-recurrent kernel when it
    does not; True takes the chunked prefill (the caller vouches for the bound); False
    the token-recurrent kernel.  When any input requires grad the call is recorded for
    autograd through the chunked prefill, whose backward (``chunk_bwd``, gradients to
    q, k, v, alpha, beta and initial_state) needs the same bound: a gate outside it
    raises ValueError."""
    grad = _needs_grad(q, k, v, alpha, beta, initial_state)
    if bounded is None:
        bounded = gate_within_chunk_bound(alpha)
    if grad:
        if not bounded:
            raise ValueError("recurrent_kda with autograd needs every alpha >= e^-5 (the chunked prefill and "
                             "its backward are defined for the bounded gate)")
        return _ChunkKDAFn.apply(q, k, v, alpha, beta, initial_state, chunk_size, float(scale))
    if bounded:
        return chunk_fwd(q, k, v, alpha, beta, initial_state=initial_state, output_final_state=True,
                         chunk_size=chunk_size, scale=scale)
    return recurrent_fwd(q, k, v, alpha, beta, initial_state=initial_state, output_final_state=True, scale=scale)
