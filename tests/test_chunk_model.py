"""The chunkwise algebra and sub-tile rescaling (numpy model) against the oracle."""
import numpy as np
import pytest

import oracle
from tests.chunk_model import _bf16, chunk_scan


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
