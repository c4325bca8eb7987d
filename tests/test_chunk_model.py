"""The chunkwise algebra and sub-tile rescaling (numpy model) against the oracle."""
import numpy as np
import pytest

import oracle
from tests.chunk_model import _bf16, chunk_scan, chunk_scan_bwd
from tests.helpers import dg_scale


def _inputs(rs, T, K, V, regime):
    q = rs.standard_normal((T, K)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rs.standard_normal((T, K)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rs.standard_normal((T, V))
    if regime == "fast":      # retention near e^-5 (the bound), large in-chunk rescales
        g = -5.0 * (1.0 / (1.0 + np.exp(-np.exp(1.0) * rs.normal(3.0, 1.0, (T, K)))))
    elif regime == "slow":
        g = -5.0 * (1.0 / (1.0 + np.exp(-np.exp(1.0) * rs.normal(-4.0, 1.0, (T, K)))))
    else:
        g = -5.0 * (1.0 / (1.0 + np.exp(-rs.standard_normal((T, K)))))
    beta = 1.0 / (1.0 + np.exp(-rs.standard_normal(T)))
    s0 = 0.1 * rs.standard_normal((K, V))
    return q, k, v, g, beta, s0


def _oracle(q, k, v, g, beta, s0):
    T, K = q.shape
    V = v.shape[1]
    o, f = oracle.scan(q[None, :, None], k[None, :, None], v[None, :, None], np.exp(g)[None, :, None],
                       beta[None, :, None], s0[None, None])
    return o[0, :, 0], f[0, 0]


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("regime", ["mid", "fast", "slow"])
def test_chunk_model_fp64_equals_scan(C, regime):
    rs = np.random.default_rng(100 + C)
    q, k, v, g, beta, s0 = _inputs(rs, 150, 32, 24, regime)
    eo, ef = _oracle(q, k, v, g, beta, s0)
    o, f = chunk_scan(q, k, v, g, beta, s0, C=C)
    np.testing.assert_allclose(o, eo, rtol=0, atol=1e-12 * np.abs(eo).max())
    np.testing.assert_allclose(f, ef, rtol=0, atol=1e-12 * np.abs(ef).max())


@pytest.mark.parametrize("regime", ["mid", "fast", "slow"])
def test_chunk_model_fp32_within_fp32_tolerance(regime):
    rs = np.random.default_rng(7)
    q, k, v, g, beta, s0 = _inputs(rs, 200, 64, 64, regime)
    eo, ef = _oracle(q, k, v, g, beta, s0)
    f32 = [x.astype(np.float32) for x in (q, k, v, g, beta, s0)]
    with np.errstate(over="raise", invalid="raise"):
        o, f = chunk_scan(*f32, C=64, precision="f32")
    for got, ref in ((o, eo), (f, ef)):
        err = np.abs(got - ref) / np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
        assert err.max() < 1e-4, err.max()


@pytest.mark.parametrize("regime", ["mid", "fast", "slow"])
@pytest.mark.parametrize("C", [32, 64])
def test_chunk_model_mixed_operands_within_bf16_tolerance(regime, C):
    """The kernel's operand precisions for bf16 inputs meet the 2e-2 rule with margin
    (inputs rounded to bf16 first, as the real inputs are)."""
    rs = np.random.default_rng(8)
    q, k, v, g, beta, s0 = _inputs(rs, 256, 128, 64, regime)
    q, k, v = (_bf16(x.astype(np.float32)).astype(np.float64) for x in (q, k, v))
    eo, ef = _oracle(q, k, v, g, beta, s0)
    f32 = [x.astype(np.float32) for x in (q, k, v, g, beta, s0)]
    with np.errstate(over="raise", invalid="raise"):
        o, f = chunk_scan(*f32, C=C, precision="mixed")
    for got, ref in ((o, eo), (f, ef)):
        err = np.abs(got - ref).max() / np.sqrt(np.mean(ref ** 2))
        assert err < 1e-2, err


# --- backward ---------------------------------------------------------------------------

def _oracle_bwd(q, k, v, g, beta, s0, do, dsT, scale):
    E = lambda x: x[None, :, None]
    r = oracle.scan_bwd(E(q), E(k), E(v), E(np.exp(g)), E(beta), E(do), s0[None, None], dsT[None, None],
                        scale=scale)
    # the chunked form differentiates with respect to g = ln alpha: dg = alpha * dalpha
    return [r[0][0, :, 0], r[1][0, :, 0], r[2][0, :, 0], r[3][0, :, 0] * np.exp(g), r[4][0, :, 0], r[5][0, 0]]


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("regime", ["mid", "fast", "slow"])
def test_chunk_model_bwd_fp64_equals_oracle(C, regime):
    rs = np.random.default_rng(200 + C)
    q, k, v, g, beta, s0 = _inputs(rs, 150, 32, 24, regime)
    do = rs.standard_normal((150, 24))
    dsT = rs.standard_normal((32, 24))
    ref = _oracle_bwd(q, k, v, g, beta, s0, do, dsT, 0.7)
    got = chunk_scan_bwd(q, k, v, g, beta, do, s0, dsT, C=C, scale=0.7)
    for name, a, b in zip("dq dk dv dg dbeta ds0".split(), got, ref):
        assert np.abs(a - b).max() <= 1e-11 * np.abs(b).max(), name


@pytest.mark.parametrize("regime", ["mid", "fast", "slow"])
def test_chunk_model_bwd_fp32_within_tolerance(regime):
    """float32 with the 16-row middle-row rescaling: no overflow near the decay bound, every
    gradient within 1e-4 (d ln alpha relative to the size of its terms, see dg_scale)."""
    rs = np.random.default_rng(5)
    q, k, v, g, beta, s0 = _inputs(rs, 200, 128, 128, regime)
    do = rs.standard_normal((200, 128))
    dsT = rs.standard_normal((128, 128))
    ref = _oracle_bwd(q, k, v, g, beta, s0, do, dsT, 0.5)
    f32 = [x.astype(np.float32) for x in (q, k, v, g, beta, do, s0, dsT)]
    with np.errstate(over="raise", invalid="raise"):
        got = chunk_scan_bwd(*f32[:6], s0=f32[6], dsT=f32[7], C=64, scale=0.5, dtype=np.float32)
    for name, a, b in zip("dq dk dv dg dbeta ds0".split(), got, ref):
        floor = np.sqrt(np.mean(b ** 2))
        if name == "dg":
            floor = max(floor, dg_scale(q, ref[0], k, ref[1]))
        err = np.abs(a - b) / np.maximum(np.abs(b), floor)
        assert err.max() < 1e-4, (name, err.max())
