"""Seeded synthetic inputs for the KDA recurrence (shared by tests and bench).

This module holds no part of the method's arithmetic: it only draws random
numbers and prepares them the way the model prepares its kernel inputs
(KDA cheat sheet, "How the inputs are produced": q and k pass through Swish
and an L2 norm, v through Swish, beta through a sigmoid; the scan itself
takes prepared vectors and performs no normalisation).  The decay logits z
are drawn raw; turning them into retention factors is the method's gate and
is done separately by the GPU library and by the oracle.

Draws use torch generators (CPU or CUDA) seeded per call, so the same seed
and device give the same tensors.  A normal "N(m, s)" in a recipe means mean
m and standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, gen, device, mean=0.0, std=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x


def _l2norm(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-6)


@dataclass
class PrefillInputs:
    """Inputs of one prefill call.  Token tensors are [B, T, H, *]."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    z: torch.Tensor                 # decay logits [B, T, H, K]
    log_scale: torch.Tensor         # A per head, float32 [H]
    beta: torch.Tensor              # float32 [B, T, H]
    initial_state: Optional[torch.Tensor]  # float32 [N, H, K, V] or None
    cu_seqlens: Optional[torch.Tensor]     # int32 [N + 1] or None
    g_min: float = -5.0
    chunk_size: int = 64
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        B, T, H, K = self.q.shape
        return B, T, H, K, self.v.shape[-1]

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1


def make_prefill(B, T, H, K, V, *, dtype=torch.bfloat16, seed=0, device="cpu",
                 qk="normal", v_kind="normal", z_mean=0.0, z_std=1.0, alog_std=0.0,
                 alog_const=0.0, beta_mean=0.0, state_std=None, seqlens=None,
                 g_min=-5.0, chunk_size=64, name="custom") -> PrefillInputs:
    """General recipe.  qk: "normal" = L2norm(N(0,1)); "silu" = L2norm(SiLU(N(0,1))).
    v_kind: "normal" = N(0,1); "silu" = SiLU(N(0,1)).  seqlens: packed lengths
    (then B must be 1 and T = sum(seqlens))."""
    gen = _gen(device, seed)
    if seqlens is not None:
        assert B == 1 and T == int(sum(seqlens))
    shp_k, shp_v = (B, T, H, K), (B, T, H, V)
    q = _normal(shp_k, gen, device)
    k = _normal(shp_k, gen, device)
    v = _normal(shp_v, gen, device)
    if qk == "silu":
        q, k = torch.nn.functional.silu(q), torch.nn.functional.silu(k)
    q, k = _l2norm(q), _l2norm(k)
    if v_kind == "silu":
        v = torch.nn.functional.silu(v)
    z = _normal(shp_k, gen, device, z_mean, z_std)
    log_scale = (_normal((H,), gen, device, 0.0, alog_std) if alog_std > 0
                 else torch.full((H,), float(alog_const), device=device))
    beta = torch.sigmoid(_normal((B, T, H), gen, device, beta_mean, 1.0))
    N = B if seqlens is None else len(seqlens)
    s0 = None
    if state_std is not None:
        s0 = _normal((N, H, K, V), gen, device, 0.0, state_std)
    cu = None
    if seqlens is not None:
        cu = torch.zeros(len(seqlens) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(list(seqlens), dtype=torch.int64), 0).to(torch.int32)
        cu = cu.to(device)
    return PrefillInputs(name=name, q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), z=z.to(dtype),
                         log_scale=log_scale.float(), beta=beta.float(), initial_state=s0,
                         cu_seqlens=cu, g_min=g_min, chunk_size=chunk_size,
                         meta=dict(seed=seed, seqlens=None if seqlens is None else list(seqlens)))


# ---- the five workloads -------------------------------------------------------------

def tiny_fp32(device="cpu", seed=1) -> PrefillInputs:
    """B=1 T=64 H=2 K=V=16 fp32; q,k L2norm(N(0,1)); v N(0,1); z N(0,1), A=0, g_min=-5;
    beta = sigmoid(N(0,1)); zero initial state."""
    return make_prefill(1, 64, 2, 16, 16, dtype=torch.float32, seed=seed, device=device,
                        name="tiny_fp32_B1_T64_H2_K16_V16")


def mixed_resume(device="cpu", seed=2) -> PrefillInputs:
    """B=2 T=1024 H=8 K=64 V=128 bf16; A ~ N(0,0.5) per head; S0 ~ N(0,0.1); chunk 64."""
    return make_prefill(2, 1024, 8, 64, 128, dtype=torch.bfloat16, seed=seed, device=device,
                        alog_std=0.5, state_std=0.1, name="mixed_resume_B2_T1024_H8_K64_V128")


def k3_prefill(device="cpu", seed=3, T=8192, H=96) -> PrefillInputs:
    """Kimi K3 KDA layer prefill: B=1 T=8192 H=96 K=V=128 bf16; q,k L2norm(SiLU(N(0,1)));
    v SiLU(N(0,1)); z N(0,1.5); A ~ N(0,0.5); g_min=-5; beta sigmoid(N(0,1)); zero state."""
    return make_prefill(1, T, H, 128, 128, dtype=torch.bfloat16, seed=seed, device=device,
                        qk="silu", v_kind="silu", z_std=1.5, alog_std=0.5,
                        name="k3_prefill_B1_T%d_H%d_K128_V128" % (T, H))


def varlen_lengths(seed=5, n=8, lo=1024, hi=32768):
    gen = _gen("cpu", seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]


def varlen_stress(device="cpu", seed=5, lengths=None, H=96) -> PrefillInputs:
    """8 packed sequences, lengths uniform in [1024, 32768]; H=96 K=V=128 bf16; q,k,v as the
    K3 prefill; z ~ N(3,1) with A=1 (retention near e^-5); beta sigmoid(N(2,1)); zero states."""
    if lengths is None:
        lengths = varlen_lengths(seed)
    T = int(sum(lengths))
    return make_prefill(1, T, H, 128, 128, dtype=torch.bfloat16, seed=seed, device=device,
                        qk="silu", v_kind="silu", z_mean=3.0, alog_const=1.0, beta_mean=2.0,
                        seqlens=lengths, name="varlen_stress_N%d_T%d_H%d" % (len(lengths), T, H))


@dataclass
class DecodeInputs:
    """Kept state plus per-step inputs for `steps` successive single-token steps."""
    name: str
    state: torch.Tensor      # float32 [B, H, K, V]
    q: torch.Tensor          # [steps, B, H, K]
    k: torch.Tensor
    v: torch.Tensor          # [steps, B, H, V]
    z: torch.Tensor          # [steps, B, H, K]
    log_scale: torch.Tensor  # [H]
    beta: torch.Tensor       # float32 [steps, B, H]
    g_min: float = -5.0


def decode(device="cpu", seed=4, B=64, H=96, K=128, V=128, steps=256,
           dtype=torch.bfloat16) -> DecodeInputs:
    """Decode: kept fp32 state ~ N(0,0.05); per step q,k L2norm(N(0,1)), v N(0,1), z N(0,1)
    with A=0, beta sigmoid(N(0,1))."""
    gen = _gen(device, seed)
    state = _normal((B, H, K, V), gen, device, 0.0, 0.05)
    q = _l2norm(_normal((steps, B, H, K), gen, device)).to(dtype)
    k = _l2norm(_normal((steps, B, H, K), gen, device)).to(dtype)
    v = _normal((steps, B, H, V), gen, device).to(dtype)
    z = _normal((steps, B, H, K), gen, device).to(dtype)
    beta = torch.sigmoid(_normal((steps, B, H), gen, device))
    return DecodeInputs(name="decode_B%d_H%d_K%d_V%d_steps%d" % (B, H, K, V, steps), state=state,
                        q=q, k=k, v=v, z=z, log_scale=torch.zeros(H, device=device), beta=beta)


def short_prompts(device="cpu", seed=6, B=64, T=16, H=96, K=128, V=128,
                  dtype=torch.bfloat16) -> PrefillInputs:
    """Short continuations over a kept state (speculative decoding / short prompts):
    B sequences of T tokens each, kept fp32 state ~ N(0,0.05), the decode workload's
    per-token recipe (q,k L2norm(N(0,1)), v N(0,1), z N(0,1) with A=0, beta sigmoid(N(0,1)))."""
    gen = _gen(device, seed)
    s0 = _normal((B, H, K, V), gen, device, 0.0, 0.05)
    q = _l2norm(_normal((B, T, H, K), gen, device)).to(dtype)
    k = _l2norm(_normal((B, T, H, K), gen, device)).to(dtype)
    v = _normal((B, T, H, V), gen, device).to(dtype)
    z = _normal((B, T, H, K), gen, device).to(dtype)
    beta = torch.sigmoid(_normal((B, T, H), gen, device))
    return PrefillInputs(name="short_prompts_B%d_T%d_H%d_K%d_V%d" % (B, T, H, K, V), q=q, k=k, v=v, z=z,
                         log_scale=torch.zeros(H, device=device), beta=beta.float(), initial_state=s0,
                         cu_seqlens=None, g_min=-5.0, chunk_size=16, meta=dict(seed=seed, seqlens=None))


def retention(shape, seed=0, device="cpu", lo_log=-5.0, hi_log=0.0) -> torch.Tensor:
    """Random retention factors drawn log-uniformly in [e^lo_log, e^hi_log] (an input
    distribution for scan-only tests, not the gate)."""
    gen = _gen(device, seed)
    u = torch.rand(shape, generator=gen, device=device, dtype=torch.float64)
    return torch.exp(lo_log + (hi_log - lo_log) * u).float()


def cotangents(B, T, H, V, K, N, seed=0, device="cpu", final=True):
    """Seeded upstream gradients for a backward call: d_out ~ N(0,1) [B,T,H,V] float32 and
    d_final_state ~ N(0,1) [N,H,K,V] float32 (None when ``final`` is False)."""
    gen = _gen(device, seed)
    d_out = _normal((B, T, H, V), gen, device)
    d_fin = _normal((N, H, K, V), gen, device) if final else None
    return d_out, d_fin
