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


# --- backward ---------------------------------------------------------------------------
# Reverse-mode derivative of the chunkwise form above, organised the way the GPU backward
# runs it: (1) per-chunk preparation (Gamma, A_kk, T, W, U, A_qk), (2) a forward pass over
# the chunks that keeps each chunk's start state h_n and pseudo-values Vt_n, (3) a
# reverse pass that keeps each chunk's end-state gradient dh_n and dVt_n,
#     dVt = Kd dS' + A_qk^T dO,   dS = gamma_C dS' + Qg^T dO - W^T dVt
# (Kd = K e^{Gamma_C - Gamma}, Qg = Q e^Gamma), and (4) per-chunk gradients:
#     dQ = (dO h^T) e^Gamma + [dA_qk K e^{..}]                 dA_qk = tril(dO Vt^T)
#     dKd = Vt dh^T,  dW = -dVt h^T,  dU = dVt,  dT = dU (beta V)^T + dW (beta K e^Gamma)^T
#     dV = beta (T^T dU),  dA = -strict_tril(T^T dT T^T),  dAbar = beta dA
#     dGamma = Q dQ + K (dK_row-side - dK_col-side), plus on the last row
#              sum_r K dK_S + gamma_C rowsum(h dh)
#     d ln alpha = reverse cumulative sum of dGamma inside the chunk.
# Every decayed product sum_c X_rc Y_sc e^{Gamma_rc - Gamma_sc} (and its two adjoints)
# is split at the middle row m of the 16-row tile of r: e^{Gamma_r - Gamma_m} and
# e^{Gamma_m - Gamma_s}, neither above e^40 when g >= -5.


def _tile_ref(Gam, p):
    return Gam[16 * p + 7]


def _decayed(Gam, X, Y, M=None, strict=False):
    """A[r, s] = sum_c X_rc Y_sc e^{Gam_rc - Gam_sc} on the (strictly) lower triangle, by
    16-row tiles of r with the exponent split at the tile's middle row."""
    C = X.shape[0]
    A = np.zeros((C, C), X.dtype)
    for p in range(C // 16):
        ri = slice(16 * p, 16 * p + 16)
        m = _tile_ref(Gam, p)
        xh = X[ri] * np.exp(Gam[ri] - m)
        yh = Y[:16 * p + 16] * np.exp(m - Gam[:16 * p + 16])
        A[ri, :16 * p + 16] = xh @ yh.T
    return np.where(np.tri(C, C, -1 if strict else 0, dtype=bool), A, 0)


def _decayed_adjoints(Gam, M, X, Y):
    """For A[r,s] = sum_c X_rc Y_sc e^{Gam_rc - Gam_sc} (r >= s) and dL/dA = M (lower):
    dX[r] = sum_s M[r,s] Y_s e^{Gam_r - Gam_s},  dY[s] = sum_r M[r,s] X_r e^{Gam_r - Gam_s}."""
    C = X.shape[0]
    dX = np.zeros_like(X)
    dY = np.zeros_like(Y)
    for p in range(C // 16):
        ri = slice(16 * p, 16 * p + 16)
        n = 16 * p + 16
        m = _tile_ref(Gam, p)
        a = np.exp(Gam[ri] - m)            # row factors of tile p
        b = np.exp(m - Gam[:n])            # column factors for s < 16p + 16
        dX[ri] = a * (M[ri, :n] @ (Y[:n] * b))
        dY[:n] += b * (M[ri, :n].T @ (X[ri] * a))
    return dX, dY


def chunk_scan_bwd(q, k, v, g, beta, do, s0=None, dsT=None, C=64, scale=1.0, dtype=np.float64):
    """Gradients of chunk_scan for L = <do, out * scale> + <dsT, S_T>, one (sequence,
    head): returns dq, dk, dv, dg (with respect to the log-decay g), dbeta, ds0."""
    f = dtype
    T, K = q.shape
    V = v.shape[1]
    NT = (T + C - 1) // C
    pad = NT * C
    def padded(x, w):
        y = np.zeros((pad, w), f)
        y[:T] = x
        return y
    Q, Kk, Vv, G, dO = padded(q, K), padded(k, K), padded(v, V), padded(g, K), padded(do, V) * f(scale)
    Bt = np.zeros(pad, f)
    Bt[:T] = beta
    # (1) per-chunk preparation
    prep = []
    for n in range(NT):
        sl = slice(n * C, n * C + C)
        Gam = np.cumsum(G[sl], axis=0, dtype=f)
        Akk = Bt[sl, None] * _decayed(Gam, Kk[sl], Kk[sl], strict=True)
        Tm = np.linalg.inv(np.eye(C, dtype=f) + Akk).astype(f)
        Tm = np.where(np.tri(C, C, 0, dtype=bool), Tm, 0)
        Aqk = _decayed(Gam, Q[sl], Kk[sl])
        gam = np.exp(Gam)
        W = Tm @ (Bt[sl, None] * Kk[sl] * gam)
        U = Tm @ (Bt[sl, None] * Vv[sl])
        Kd = Kk[sl] * np.exp(Gam[C - 1] - Gam)
        Qg = Q[sl] * gam
        prep.append((Gam, Tm, Aqk, W, U, Kd, Qg, gam[C - 1]))
    # (2) forward over chunks
    S = np.zeros((K, V), f) if s0 is None else s0.astype(f).copy()
    h, Vt = [], []
    for n in range(NT):
        Gam, Tm, Aqk, W, U, Kd, Qg, gC = prep[n]
        h.append(S.copy())
        vt = U - W @ S
        Vt.append(vt)
        S = gC[:, None] * S + Kd.T @ vt
    # (3) reverse over chunks
    dS = np.zeros((K, V), f) if dsT is None else dsT.astype(f).copy()
    dh, dVt = [None] * NT, [None] * NT
    for n in range(NT - 1, -1, -1):
        Gam, Tm, Aqk, W, U, Kd, Qg, gC = prep[n]
        sl = slice(n * C, n * C + C)
        dh[n] = dS.copy()
        dvt = Kd @ dS + Aqk.T @ dO[sl]
        dVt[n] = dvt
        dS = gC[:, None] * dS + Qg.T @ dO[sl] - W.T @ dvt
    ds0 = dS
    # (4) per-chunk gradients
    dq, dk, dg = (np.zeros((pad, K), f) for _ in range(3))
    dv = np.zeros((pad, V), f)
    db = np.zeros(pad, f)
    for n in range(NT):
        Gam, Tm, Aqk, W, U, Kd, Qg, gC = prep[n]
        sl = slice(n * C, n * C + C)
        Qc, Kc, Vc, Bc, dOc = Q[sl], Kk[sl], Vv[sl], Bt[sl], dO[sl]
        gam = np.exp(Gam)
        dQ = (dOc @ h[n].T) * gam
        dAqk = np.where(np.tri(C, C, 0, dtype=bool), dOc @ Vt[n].T, 0)
        dQA, dKA = _decayed_adjoints(Gam, dAqk, Qc, Kc)
        dQ += dQA
        dKS = (Vt[n] @ dh[n].T) * np.exp(Gam[C - 1] - Gam)
        dW = -dVt[n] @ h[n].T
        dU = dVt[n]
        Bk = Bc[:, None] * Kc * gam
        dT = dU @ (Bc[:, None] * Vc).T + dW @ Bk.T
        dBv = Tm.T @ dU
        dBk = Tm.T @ dW
        dV = Bc[:, None] * dBv
        dbeta = np.sum(Vc * dBv, axis=1) + np.sum(Kc * gam * dBk, axis=1)
        dKW = Bc[:, None] * gam * dBk
        dA = np.where(np.tri(C, C, -1, dtype=bool), -(Tm.T @ dT @ Tm.T), 0)
        Abar = _decayed(Gam, Kc, Kc, strict=True)
        dbeta += np.sum(dA * Abar, axis=1)
        dK1, dK2 = _decayed_adjoints(Gam, Bc[:, None] * dA, Kc, Kc)
        dK = dKA + dKS + dKW + dK1 + dK2
        dGam = Qc * dQ + Kc * (dK1 + dKW - dKA - dK2)
        # the end-of-chunk terms reach every row's log-decay: gamma_C rowsum(h dh) and,
        # from Kd = K e^{Gamma_C - Gamma_r}, the rows before r (sum_{r' < r} K dK_S),
        # summed forwards rather than as a difference of two reverse sums
        eS = Kc * dKS
        dlog = np.cumsum(dGam[::-1], axis=0)[::-1] + gC * np.sum(h[n] * dh[n], axis=1)
        dlog[1:] += np.cumsum(eS, axis=0)[:-1]
        dq[sl], dk[sl], dv[sl], dg[sl], db[sl] = dQ, dK, dV, dlog, dbeta
    return dq[:T] * f(1), dk[:T], dv[:T], dg[:T], db[:T], ds0
