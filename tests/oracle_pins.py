"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each function takes an ``oracle.Oracle`` handle and raises AssertionError when
the handle disagrees with the pin.  ``test_oracle_pins.py`` runs them against
the real oracle, and against deliberately broken copies of its C source to
show that each plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_inputs(rs, B, T, H, K, V, unit_keys=True):
    q = rs.standard_normal((B, T, H, K))
    k = rs.standard_normal((B, T, H, K))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rs.standard_normal((B, T, H, V))
    alpha = np.exp(rs.uniform(-5.0, 0.0, (B, T, H, K)))
    beta = rs.uniform(0.0, 1.0, (B, T, H))
    s0 = 0.3 * rs.standard_normal((B, H, K, V))
    return q, k, v, alpha, beta, s0


# --- recurrence pins -----------------------------------------------------------------

def pin_toy_memory(orc):
    """Worked example of the PaperLeet page ('Toy experiment'): exact outputs."""
    with open(os.path.join(GOLDEN, "toy_memory.json")) as f:
        g = json.load(f)
    T, K, V = len(g["values"]), g["K"], g["V"]
    k = np.array(g["keys"], float).reshape(1, T, 1, K)
    q = np.array(g["queries"], float).reshape(1, T, 1, K)
    v = np.array(g["values"], float).reshape(1, T, 1, V)
    a = np.array(g["alpha"], float).reshape(1, T, 1, K)
    b = np.array(g["beta"], float).reshape(1, T, 1)
    o, _ = orc.scan(q, k, v, a, b)
    assert np.array_equal(o.reshape(-1), np.array(g["expected_outputs"], float)), o.reshape(-1)


def pin_empty_sequence(orc):
    """Contract table, 'Empty sequence': T=0 gives a zero-length output and final state
    equal to the supplied state, or zeros."""
    rs = np.random.default_rng(10)
    B, H, K, V = 2, 3, 4, 5
    z = np.zeros((B, 0, H, K))
    s0 = rs.standard_normal((B, H, K, V))
    o, f = orc.scan(z, z, np.zeros((B, 0, H, V)), z, np.zeros((B, 0, H)), s0)
    assert o.shape == (B, 0, H, V)
    assert np.array_equal(f, s0)
    o, f = orc.scan(z, z, np.zeros((B, 0, H, V)), z, np.zeros((B, 0, H)))
    assert np.array_equal(f, np.zeros((B, H, K, V)))


def pin_exact_recall(orc):
    """alpha=1, beta=1 and orthonormal keys: k_i^T k_j = delta_ij, so each write stores v_j
    under k_j without disturbing the others and querying k_j returns v_j."""
    rs = np.random.default_rng(11)
    K, V, n = 8, 6, 5
    basis, _ = np.linalg.qr(rs.standard_normal((K, K)))
    keys = basis[:n]
    vals = rs.standard_normal((n, V))
    T = 2 * n
    k = np.zeros((1, T, 1, K)); q = np.zeros((1, T, 1, K)); v = np.zeros((1, T, 1, V))
    b = np.zeros((1, T, 1)); a = np.ones((1, T, 1, K))
    k[0, :n, 0] = keys; v[0, :n, 0] = vals; b[0, :n, 0] = 1.0; q[0, :n, 0] = keys
    k[0, n:, 0] = keys[::-1]            # no write (beta = 0) on the read-back tokens
    q[0, n:, 0] = keys[::-1]
    o, _ = orc.scan(q, k, v, a, b)
    np.testing.assert_allclose(o[0, n:, 0], vals[::-1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, :n, 0], vals, rtol=0, atol=1e-12)


def pin_overwrite(orc):
    """Cheat sheet lineage table, DeltaNet row: under the delta rule a second write to the
    same unit key overwrites the first; reading that key returns the second value."""
    K, V = 4, 3
    key = np.array([0.5, 0.5, 0.5, 0.5])
    k = np.tile(key, (1, 3, 1, 1)); q = k.copy()
    v = np.array([[1.0, -2.0, 3.0], [4.0, 5.0, -6.0], [0.0, 0.0, 0.0]]).reshape(1, 3, 1, V)
    b = np.array([1.0, 1.0, 0.0]).reshape(1, 3, 1)
    o, _ = orc.scan(q, k, v, np.ones((1, 3, 1, K)), b)
    np.testing.assert_allclose(o[0, 1, 0], v[0, 1, 0], atol=1e-14)
    np.testing.assert_allclose(o[0, 2, 0], v[0, 1, 0], atol=1e-14)


def pin_zero_writes(orc):
    """beta = 0: no correction ever happens, so S_t = Diag(prod_{r<=t} alpha_r) S_0 and
    o_t = S_t^T q_t in closed form."""
    rs = np.random.default_rng(12)
    B, T, H, K, V = 2, 9, 2, 5, 4
    q, k, v, alpha, _, s0 = _rand_inputs(rs, B, T, H, K, V)
    o, f = orc.scan(q, k, v, alpha, np.zeros((B, T, H)), s0)
    cum = np.cumprod(alpha, axis=1)                              # [B,T,H,K]
    exp_o = np.einsum("bthk,bhkv,bthk->bthv", cum, s0, q)
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f, cum[:, -1, :, :, None] * s0, rtol=1e-12, atol=1e-14)


def literal_matrix_scan(q, k, v, alpha, beta, s0, scale=1.0):
    """Cheat sheet 'The recurrence': S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T,
    o_t = S_t^T q_t, evaluated with explicit K x K matrices (a different formula from the
    oracle's fade / predict / correct loop)."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    out = np.zeros((B, T, H, V))
    fin = np.zeros((B, H, K, V))
    eye = np.eye(K)
    for b in range(B):
        for h in range(H):
            S = s0[b, h].copy()
            for t in range(T):
                kt = k[b, t, h][:, None]
                S = (eye - beta[b, t, h] * kt @ kt.T) @ np.diag(alpha[b, t, h]) @ S \
                    + beta[b, t, h] * kt @ v[b, t, h][None, :]
                out[b, t, h] = scale * (S.T @ q[b, t, h])
            fin[b, h] = S
    return out, fin


def pin_literal_matrix_form(orc):
    """Cheat sheet erase/fade/write form equals the contract's fade/correct/read form."""
    rs = np.random.default_rng(13)
    q, k, v, alpha, beta, s0 = _rand_inputs(rs, 2, 7, 2, 5, 3)
    o, f = orc.scan(q, k, v, alpha, beta, s0, scale=0.75)
    eo, ef = literal_matrix_scan(q, k, v, alpha, beta, s0, scale=0.75)
    np.testing.assert_allclose(o, eo, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f, ef, rtol=1e-11, atol=1e-12)
    # non-unit keys and beta outside (0,1) are still the same algebra
    q, k, v, alpha, beta, s0 = _rand_inputs(rs, 1, 6, 1, 4, 4, unit_keys=False)
    o, f = orc.scan(q, k, v, alpha, 0.3 * beta, s0)
    eo, ef = literal_matrix_scan(q, k, v, alpha, 0.3 * beta, s0)
    np.testing.assert_allclose(o, eo, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(f, ef, rtol=1e-10, atol=1e-11)


def pin_gated_deltanet(orc):
    """Lineage table, Gated DeltaNet row: one scalar rate per head.  With alpha_t uniform
    over channels the update is alpha_t (I - beta k k^T) S + beta k v^T."""
    rs = np.random.default_rng(14)
    B, T, H, K, V = 1, 8, 1, 4, 3
    q, k, v, _, beta, s0 = _rand_inputs(rs, B, T, H, K, V)
    a_scalar = rs.uniform(0.2, 1.0, (B, T, H))
    alpha = np.repeat(a_scalar[..., None], K, axis=-1)
    o, f = orc.scan(q, k, v, alpha, beta, s0)
    S = s0[0, 0].copy()
    for t in range(T):
        kt = k[0, t, 0][:, None]
        S = a_scalar[0, t, 0] * (np.eye(K) - beta[0, t, 0] * kt @ kt.T) @ S + beta[0, t, 0] * kt @ v[0, t, 0][None]
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[0, t, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f[0, 0], S, rtol=1e-12, atol=1e-13)


def pin_segmented_continuation(orc):
    """Contract: the returned state continues the scan.  Splitting at an unaligned point and
    resuming from the returned state gives the one-call result."""
    rs = np.random.default_rng(15)
    q, k, v, alpha, beta, s0 = _rand_inputs(rs, 2, 23, 2, 6, 5)
    o, f = orc.scan(q, k, v, alpha, beta, s0)
    t1 = 9
    o1, f1 = orc.scan(q[:, :t1], k[:, :t1], v[:, :t1], alpha[:, :t1], beta[:, :t1], s0)
    o2, f2 = orc.scan(q[:, t1:], k[:, t1:], v[:, t1:], alpha[:, t1:], beta[:, t1:], f1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(f2, f, rtol=1e-13, atol=1e-14)


def pin_causal_prefix(orc):
    """Outputs up to t do not depend on any input after t (bitwise)."""
    rs = np.random.default_rng(16)
    q, k, v, alpha, beta, s0 = _rand_inputs(rs, 1, 12, 2, 4, 4)
    o, _ = orc.scan(q, k, v, alpha, beta, s0)
    t = 5
    q2, k2, v2, a2, b2 = (x.copy() for x in (q, k, v, alpha, beta))
    for x in (q2, k2, v2):
        x[:, t + 1:] = rs.standard_normal(x[:, t + 1:].shape)
    a2[:, t + 1:] = rs.uniform(0.1, 1, a2[:, t + 1:].shape)
    b2[:, t + 1:] = rs.uniform(0, 1, b2[:, t + 1:].shape)
    o2, _ = orc.scan(q2, k2, v2, a2, b2, s0)
    assert np.array_equal(o[:, :t + 1], o2[:, :t + 1])
    assert not np.array_equal(o[:, t + 1:], o2[:, t + 1:])


def pin_varlen_equals_separate(orc):
    """Packed sequences (cu_seqlens) restart the state per sequence: a packed call equals
    separate calls, including a zero-length sequence (final = its initial state)."""
    rs = np.random.default_rng(17)
    lens = [5, 0, 11, 3]
    T = sum(lens)
    H, K, V = 2, 4, 3
    q, k, v, alpha, beta, _ = _rand_inputs(rs, 1, T, H, K, V)
    s0 = rs.standard_normal((len(lens), H, K, V))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, f = orc.scan(q, k, v, alpha, beta, s0, cu_seqlens=cu)
    for s, (a0, a1) in enumerate(zip(cu[:-1], cu[1:])):
        sl = slice(a0, a1)
        os_, fs = orc.scan(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl], s0[s:s + 1])
        assert np.array_equal(o[:, sl], os_)
        assert np.array_equal(f[s], fs[0])


def pin_scale_is_linear(orc):
    """The read is o_t = scale * S_t^T q_t: the state does not depend on scale and the
    output is linear in it (scale 1 = the contract's unscaled read)."""
    rs = np.random.default_rng(18)
    q, k, v, alpha, beta, s0 = _rand_inputs(rs, 1, 6, 1, 4, 3)
    o1, f1 = orc.scan(q, k, v, alpha, beta, s0, scale=1.0)
    o2, f2 = orc.scan(q, k, v, alpha, beta, s0, scale=0.125)
    assert np.array_equal(f1, f2)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-15, atol=0)


# --- gate pins -------------------------------------------------------------------------

def pin_gate_closed_forms(orc):
    """PaperLeet 'Formula and conventions': g = g_min sigmoid(e^A z), alpha = e^g.
    z = 0 gives sigmoid = 1/2 exactly, so alpha = e^{g_min/2}; the Fig. 3(a) setting
    (A = 0, g_min = -5, logits -10..10) reduces to the textbook logistic function,
    taken here from scipy.special.expit."""
    H, K = 1, 5
    z = np.array([-10.0, -1.0, 0.0, 1.0, 10.0]).reshape(1, H, K)
    a = orc.bounded_decay(z, np.zeros(H), g_min=-5.0)
    assert abs(a[0, 0, 2] - math.exp(-2.5)) <= 1e-15
    g = orc.bounded_decay(z, np.zeros(H), g_min=-5.0, out_log=True)
    np.testing.assert_allclose(g.reshape(-1), -5.0 * expit(z.reshape(-1)), rtol=1e-14)
    assert abs(g[0, 0, 0] - (-2.2699e-4)) < 1e-8 and abs(g[0, 0, 4] - (-4.99977)) < 1e-5
    np.testing.assert_allclose(np.log(a), g, rtol=1e-12, atol=1e-16)


def pin_gate_scale_and_bias(orc):
    """The per-head scale is e^A applied to (z + bias): g(A=ln s, z) = g(A=0, s z) and a
    bias b acts as z + b (KDARecurrent 'Decay and write strength': dt_bias is added to the
    gate input, then the positive e^A is broadcast per head)."""
    rs = np.random.default_rng(19)
    H, K = 3, 6
    z = rs.standard_normal((4, H, K))
    A = np.array([math.log(2.0), -0.7, 0.3])
    bias = rs.standard_normal((H, K))
    got = orc.bounded_decay(z, A, g_min=-3.0, bias=bias, out_log=True)
    ref = orc.bounded_decay(np.exp(A)[None, :, None] * (z + bias[None]), np.zeros(H), g_min=-3.0,
                            out_log=True)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(got, -3.0 * expit(np.exp(A)[None, :, None] * (z + bias[None])),
                               rtol=1e-13)


def pin_gate_range_and_limits(orc):
    """Cheat sheet gate table: alpha lies in (e^{g_min}, 1); floating point reaches the
    endpoints (the contract accepts them), never crosses them, and alpha is monotone
    non-increasing in z.  Extreme logits stay finite (no exp overflow)."""
    z = np.linspace(-60.0, 60.0, 2001).reshape(-1, 1, 1)
    a = orc.bounded_decay(z, np.zeros(1), g_min=-5.0).reshape(-1)
    assert np.all(np.isfinite(a))
    assert np.all(a <= 1.0) and np.all(a >= math.exp(-5.0) * (1 - 1e-15))
    assert np.all(np.diff(a) <= 0)
    ext = orc.bounded_decay(np.array([-1e4, 1e4]).reshape(2, 1, 1), np.zeros(1), g_min=-5.0).reshape(-1)
    assert ext[0] == 1.0 and abs(ext[1] - math.exp(-5.0)) < 1e-16


# --- gradient pins ---------------------------------------------------------------------
# PaperLeet "Return requirements": gradients reach q, k, v, alpha, beta and the initial
# state through the scan, and logits and log_scale through bounded_decay.  The backward
# functions are pinned to central differences of the forward functions (themselves
# pinned above), element by element, and to closed forms.

def _central_differences(f, arrays, eps=1e-6):
    """d f / d x for every element of every array in ``arrays`` (modified in place and
    restored), by (f(x + eps) - f(x - eps)) / (2 eps)."""
    out = []
    for a in arrays:
        g = np.zeros_like(a)
        flat, gf = a.reshape(-1), g.reshape(-1)
        for i in range(flat.size):
            x0 = flat[i]
            flat[i] = x0 + eps
            fp = f()
            flat[i] = x0 - eps
            fm = f()
            flat[i] = x0
            gf[i] = (fp - fm) / (2 * eps)
        out.append(g)
    return out


def _assert_grads_close(got, ref, names, tol=1e-7):
    for g, r, n in zip(got, ref, names):
        assert g.shape == r.shape, (n, g.shape, r.shape)
        err = np.max(np.abs(g - r) / np.maximum(1.0, np.abs(r))) if g.size else 0.0
        assert err <= tol, "%s: gradient differs from central differences by %g" % (n, err)


def pin_bwd_finite_differences(orc):
    """Every gradient of the scan, element by element, against central differences of
    L = <d_out, out> + <d_final, final_state>, with an initial state and a read scale."""
    rs = np.random.default_rng(30)
    B, T, H, K, V = 2, 6, 2, 3, 2
    q, k, v, alpha, beta, s0 = _rand_inputs(rs, B, T, H, K, V)
    alpha = rs.uniform(0.3, 1.0, alpha.shape)
    do = rs.standard_normal((B, T, H, V))
    dsT = rs.standard_normal((B, H, K, V))
    scale = 0.8

    def loss():
        o, f = orc.scan(q, k, v, alpha, beta, s0, scale=scale)
        return float(np.sum(do * o) + np.sum(dsT * f))
    got = orc.scan_bwd(q, k, v, alpha, beta, do, s0, dsT, scale=scale)
    ref = _central_differences(loss, [q, k, v, alpha, beta, s0])
    _assert_grads_close(got, ref, ["dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state"])


def pin_bwd_finite_differences_varlen(orc):
    """Packed sequences with an empty one, no initial state (its gradient is taken at the
    zero state), no final-state gradient, and gates at the endpoints alpha in {0, 1},
    beta in {0, 1} that the contract accepts."""
    rs = np.random.default_rng(31)
    cu = np.array([0, 3, 3, 8])
    T, H, K, V = 8, 1, 2, 3
    q, k, v, alpha, beta, _ = _rand_inputs(rs, 1, T, H, K, V, unit_keys=False)
    alpha[0, 1, 0, 0] = 0.0
    alpha[0, 4, 0, 1] = 1.0
    alpha[0, 5] = 1.0
    beta[0, 2, 0] = 0.0
    beta[0, 6, 0] = 1.0
    do = rs.standard_normal((1, T, H, V))
    zero = np.zeros((3, H, K, V))

    def loss():
        o, _ = orc.scan(q, k, v, alpha, beta, zero, cu_seqlens=cu)
        return float(np.sum(do * o))
    got = orc.scan_bwd(q, k, v, alpha, beta, do, None, None, cu_seqlens=cu)
    ref = _central_differences(loss, [q, k, v, alpha, beta, zero])
    _assert_grads_close(got, ref, ["dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state"])


def pin_bwd_single_token(orc):
    """One token from a state S0: o = scale S_1^T q with S_1 = Diag(a) S0 + b k (v - k^T Diag(a) S0)^T.
    From S0 = 0, o = scale b (k.q) v, so dq = scale b (v.do) k, dk = scale b (v.do) q,
    dv = scale b (k.q) do, dbeta = scale (k.q)(v.do), dalpha = 0, and
    dS0 = Diag(a) (I - b k k^T) scale q do^T."""
    rs = np.random.default_rng(32)
    K, V, scale = 4, 3, 0.6
    q, k, v, alpha, beta, _ = _rand_inputs(rs, 1, 1, 1, K, V, unit_keys=False)
    do = rs.standard_normal((1, 1, 1, V))
    dq, dk, dv, da, db, ds0 = orc.scan_bwd(q, k, v, alpha, beta, do, None, None, scale=scale)
    qq, kk, vv, aa, bb, dd = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], alpha[0, 0, 0], beta[0, 0, 0], do[0, 0, 0]
    tol = dict(rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dq[0, 0, 0], scale * bb * (vv @ dd) * kk, **tol)
    np.testing.assert_allclose(dk[0, 0, 0], scale * bb * (vv @ dd) * qq, **tol)
    np.testing.assert_allclose(dv[0, 0, 0], scale * bb * (kk @ qq) * dd, **tol)
    np.testing.assert_allclose(db[0, 0, 0], scale * (kk @ qq) * (vv @ dd), **tol)
    assert np.all(da == 0.0)
    dS1 = scale * np.outer(qq, dd)
    np.testing.assert_allclose(ds0[0, 0], aa[:, None] * ((np.eye(K) - bb * np.outer(kk, kk)) @ dS1), **tol)


def pin_bwd_empty_sequence(orc):
    """T = 0: no token gradients, and the final state's gradient passes straight through
    to the initial state (final = initial for an empty scan)."""
    rs = np.random.default_rng(33)
    B, H, K, V = 2, 2, 3, 4
    z = np.zeros((B, 0, H, K))
    dsT = rs.standard_normal((B, H, K, V))
    res = orc.scan_bwd(z, z, np.zeros((B, 0, H, V)), z, np.zeros((B, 0, H)), np.zeros((B, 0, H, V)),
                       rs.standard_normal((B, H, K, V)), dsT)
    assert res[0].shape == (B, 0, H, K) and res[2].shape == (B, 0, H, V)
    assert np.array_equal(res[5], dsT)


def pin_bwd_gate_finite_differences(orc):
    """Gradients of bounded_decay into the logits, the per-head log-scale and the bias,
    for a loss on alpha and on g = ln alpha, against central differences."""
    rs = np.random.default_rng(34)
    rows, H, K, gmin = 3, 2, 3, -4.0
    z = rs.standard_normal((rows, H, K))
    A = rs.standard_normal(H) * 0.5
    bias = rs.standard_normal((H, K))
    w = rs.standard_normal((rows, H, K))
    for as_log in (False, True):
        def loss():
            return float(np.sum(w * orc.bounded_decay(z, A, g_min=gmin, bias=bias, out_log=as_log)))
        got = orc.bounded_decay_bwd(z, A, w, g_min=gmin, bias=bias, grad_is_log=as_log)
        ref = _central_differences(loss, [z, A, bias])
        _assert_grads_close(got, ref, ["dz", "dlog_scale", "dbias"])


def pin_bwd_gate_closed_form(orc):
    """At z + bias = 0 the sigmoid is 1/2 with slope 1/4, so alpha = e^{g_min/2} and
    dL/dz = w alpha g_min e^A / 4; the log-scale receives nothing (x = 0)."""
    H, K, gmin = 2, 3, -5.0
    A = np.array([0.0, math.log(3.0)])
    w = np.arange(1.0, 1.0 + 2 * H * K).reshape(2, H, K)
    dz, dls, db = orc.bounded_decay_bwd(np.zeros((2, H, K)), A, w, g_min=gmin)
    ref = w * math.exp(gmin / 2) * gmin * np.exp(A)[None, :, None] / 4
    np.testing.assert_allclose(dz, ref, rtol=1e-14)
    assert np.all(dls == 0.0)
    np.testing.assert_allclose(db, dz.sum(axis=0), rtol=1e-14)


RECURRENCE_PINS = [pin_toy_memory, pin_empty_sequence, pin_exact_recall, pin_overwrite,
                   pin_zero_writes, pin_literal_matrix_form, pin_gated_deltanet,
                   pin_segmented_continuation, pin_causal_prefix, pin_varlen_equals_separate,
                   pin_scale_is_linear]
GATE_PINS = [pin_gate_closed_forms, pin_gate_scale_and_bias, pin_gate_range_and_limits]
GRADIENT_PINS = [pin_bwd_finite_differences, pin_bwd_finite_differences_varlen, pin_bwd_single_token,
                 pin_bwd_empty_sequence, pin_bwd_gate_finite_differences, pin_bwd_gate_closed_form]
ALL_PINS = RECURRENCE_PINS + GATE_PINS + GRADIENT_PINS
