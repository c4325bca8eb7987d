"""Numpy model of the chunkwise evaluation the GPU prefill kernel performs.

Test-only, and neither the oracle nor the GPU path: it checks on the CPU that
the chunkwise algebra and the 16-row sub-tile rescaling reproduce the
token-by-token recurrence, in float64 and in the kernel's working precisions.

Chunkwise form (KDA cheat sheet, "Chunkwise parallel form"; the UT transform
it names is derived here): within a chunk of C tokens with start state S and
inclusive in-chunk cumulative log-decay Gamma_i = sum_{r<=i} g_r,
    A_kk[i,j] = beta_i sum_c k_ic k_jc e^{Gamma_ic - Gamma_jc}   (j < i)
    T = (I + A_kk)^{-1}
    W = T (beta * e^Gamma * K),  U = T (beta * V),   Vt = U - W S
    A_qk[i,j] = sum_c q_ic k_jc e^{Gamma_ic - Gamma_jc}          (j <= i)
    O = (e^Gamma * Q) S + A_qk Vt
    S' = e^{Gamma_C} * S + (K * e^{Gamma_C - Gamma})^T Vt
The exponent differences are split per 16-row tile so that no factor exceeds
e^80 when every g >= -5 (cheat sheet gate table: per-tile cumulative
log-decay in (-80, 0)).
"""
from __future__ import annotations

import numpy as np


def _bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def _mm_plain(rnd):
    return lambda a, b: rnd(a) @ rnd(b)


def _mm_split(rnd):
    """hi*hi + hi*lo + lo*hi with hi = rnd(x), lo = rnd(x - hi)."""
    def mm(a, b):
        ah, bh = rnd(a), rnd(b)
        return ah @ bh + ah @ rnd(b - bh) + rnd(a - ah) @ bh
    return mm


def products(precision):
    """Operand rounding of each matrix product.  "mixed" is the GPU kernel's choice for
    bf16 inputs: bf16 for the decay-rescaled operands of A_kk, hi+lo bf16 splits for
    A_qk, fp16 for every other product."""
    names = ("Akk", "Aqk", "W", "U", "Vt", "O1", "O2", "S")
    if precision in ("f64", "f32"):
        return {n: (lambda a, b: a @ b) for n in names}
    if precision == "bf16":
        return {n: _mm_plain(_bf16) for n in names}
    if precision == "mixed":
        mm = {n: _mm_plain(_f16) for n in names}
        mm["Akk"] = _mm_plain(_bf16)
        mm["Aqk"] = _mm_split(_bf16)
        return mm
    raise ValueError(precision)


def chunk_scan(q, k, v, g, beta, s0=None, C=64, precision="f64"):
    """q,k [T,K]; v [T,V]; g [T,K] log-decay; beta [T]; one (sequence, head).
    precision: "f64", "f32", "bf16" (every operand bf16) or "mixed" (the kernel's)."""
    T, K = q.shape
    V = v.shape[1]
    f = np.float64 if precision == "f64" else np.float32
    mm = products(precision)
    S = np.zeros((K, V), f) if s0 is None else s0.astype(f).copy()
    out = np.zeros((T, V), f)
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        Q = np.zeros((C, K), f); Kc = np.zeros((C, K), f); Vc = np.zeros((C, V), f)
        G = np.zeros((C, K), f); Bt = np.zeros((C,), f)
        Q[:n], Kc[:n], Vc[:n], G[:n], Bt[:n] = q[c0:c0 + n], k[c0:c0 + n], v[c0:c0 + n], g[c0:c0 + n], beta[c0:c0 + n]
        Gam = np.cumsum(G, axis=0, dtype=f)
        P = C // 16
        R = [np.zeros(K, f) if p == 0 else Gam[16 * p - 1] for p in range(P)]
        E = [Gam[16 * p + 15] for p in range(P)]
        GC = Gam[C - 1]
        Lq = np.zeros((C, K), f); Lk = np.zeros((C, K), f); Rdg = np.zeros((C, K), f); Ro = np.zeros((C, K), f)
        Qt = np.zeros((C, K), f); Bw = np.zeros((C, K), f); Kt = np.zeros((C, K), f)
        for p in range(P):
            sl = slice(16 * p, 16 * p + 16)
            a = np.exp(Gam[sl] - R[p])                  # <= 1
            b = np.exp(R[p] - Gam[sl])                  # in [1, e^80]
            Lq[sl] = Q[sl] * a
            Lk[sl] = Bt[sl, None] * Kc[sl] * a
            Rdg[sl] = Kc[sl] * b
            Ro[sl] = Rdg[sl] * np.exp(E[p] - R[p])      # k e^{E_p - Gamma} <= 1
            Qt[sl] = Lq[sl] * np.exp(R[p])              # q e^Gamma
            Bw[sl] = Lk[sl] * np.exp(R[p])              # beta k e^Gamma
            Kt[sl] = Ro[sl] * np.exp(GC - E[p])         # k e^{Gamma_C - Gamma}
        Akk = np.zeros((C, C), f); Aqk = np.zeros((C, C), f)
        for p in range(P):
            ri = slice(16 * p, 16 * p + 16)
            for qq in range(p + 1):
                cj = slice(16 * qq, 16 * qq + 16)
                right = Rdg[cj] if qq == p else Ro[cj] * np.exp(R[p] - E[qq])
                Akk[ri, cj] = mm["Akk"](Lk[ri], right.T)
                Aqk[ri, cj] = mm["Aqk"](Lq[ri], right.T)
        Akk = np.where(np.tri(C, C, -1, dtype=bool), Akk, 0)
        Aqk = np.where(np.tri(C, C, 0, dtype=bool), Aqk, 0)
        Tm = np.linalg.inv(np.eye(C, dtype=f) + Akk).astype(f)
        Tm = np.where(np.tri(C, C, 0, dtype=bool), Tm, 0)
        W = mm["W"](Tm, Bw)
        U = mm["U"](Tm, Bt[:, None] * Vc)
        Vt = U - mm["Vt"](W, S)
        O = mm["O1"](Qt, S) + mm["O2"](Aqk, Vt)
        S = np.exp(GC)[:, None] * S + mm["S"](Kt.T, Vt)
        out[c0:c0 + n] = O[:n]
    return out, S
