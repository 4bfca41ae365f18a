"""Pins of the oracle's compensated decode attention (ResServe abstract: the FP4
activation base plus FP4 residue applied to decode attention). The oracle composes
the pinned quantizer and product with an FP32 softmax; these tests tie the whole to
results fixed from outside it: closed forms where the probabilities are exact, and
the precision gain of the residue against FP64 attention on the dequantized cache."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module", autouse=True)
def _lib():
    oracle.lib()


def _exact(q, kd, vd, H, T, D):
    """FP64 attention with unquantized q and p over the dequantized caches."""
    o = np.zeros((H, D))
    for h in range(H):
        s = q[h].astype(np.float64) @ kd[h * T:(h + 1) * T].T / np.sqrt(D)
        e = np.exp(s - s.max())
        o[h] = (e / e.sum()) @ vd[h * D:(h + 1) * D].T
    return o


@pytest.mark.parametrize("compensate", [True, False])
def test_uniform_scores_give_the_cache_mean(compensate):
    """Identical K rows: every score is equal, p = 1/T (T a power of two, exact in
    FP32), and o is the mean of the dequantized V over the tokens."""
    rng = np.random.default_rng(1)
    H, T, D = 2, 64, 32
    q = rng.standard_normal((H, D)).astype(np.float32)
    krow = rng.standard_normal((1, D)).astype(np.float32)
    k = np.repeat(krow, H * T, axis=0)
    vt = rng.standard_normal((H * D, T)).astype(np.float32)
    kq, vq = oracle.quantize(k), oracle.quantize(vt)
    o, p = oracle.decode_attention(q, kq, vq, H, T, D, compensate, return_p=True)
    assert np.all(p == np.float32(1.0 / T))
    vd = oracle.dequantize(vq)
    want = vd.reshape(H, D, T).mean(axis=2)
    np.testing.assert_allclose(o, want, rtol=1e-6, atol=1e-12)


@pytest.mark.parametrize("compensate", [True, False])
def test_one_dominant_token_selects_its_value(compensate):
    """One token's score exceeds the others by far more than FP32 exp can span: p is
    one-hot and o is that token's dequantized V column (the quantized 1.0 is exact to
    FP32 rounding of the tensor scale)."""
    rng = np.random.default_rng(2)
    H, T, D, hot = 2, 48, 32, 37
    q = np.zeros((H, D), np.float32)
    q[:, 0] = 64.0
    k = np.zeros((H * T, D), np.float32)
    k[[h * T + hot for h in range(H)], 0] = 64.0
    vt = rng.standard_normal((H * D, T)).astype(np.float32)
    kq, vq = oracle.quantize(k), oracle.quantize(vt)
    o, p = oracle.decode_attention(q, kq, vq, H, T, D, compensate, return_p=True)
    onehot = np.zeros(T, np.float32)
    onehot[hot] = 1.0
    assert np.array_equal(p, np.tile(onehot, (H, 1)))
    vd = oracle.dequantize(vq).reshape(H, D, T)
    np.testing.assert_allclose(o, vd[:, :, hot], rtol=1e-6, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_residue_recovers_precision(seed):
    """Against FP64 attention with unquantized activations, the compensated result is
    an order of magnitude closer than the uncompensated one (a residue dropped, added
    with the wrong sign or paired with the wrong cache columns loses that)."""
    rng = np.random.default_rng(seed)
    H, T, D = 3, 128, 64
    q = rng.standard_normal((H, D)).astype(np.float32)
    k = rng.standard_normal((H * T, D)).astype(np.float32)
    vt = rng.standard_normal((H * D, T)).astype(np.float32)
    kq, vq = oracle.quantize(k), oracle.quantize(vt)
    ref = _exact(q, oracle.dequantize(kq), oracle.dequantize(vq), H, T, D)
    amax = np.abs(ref).max()
    e1 = np.abs(oracle.decode_attention(q, kq, vq, H, T, D, True) - ref).max() / amax
    e0 = np.abs(oracle.decode_attention(q, kq, vq, H, T, D, False) - ref).max() / amax
    assert e1 < 0.03 and e1 < 0.15 * e0, (e1, e0)


def test_softmax_is_a_distribution_with_the_scores_order():
    rng = np.random.default_rng(6)
    s = (rng.standard_normal(1000) * 5).astype(np.float32)
    p = oracle.softmax_f32(s)
    assert p.dtype == np.float32 and np.all(p >= 0)
    assert abs(float(np.sum(p, dtype=np.float64)) - 1.0) < 1e-5
    assert np.argmax(p) == np.argmax(s)
    # shift invariance: the same probabilities for s + c (c exact in FP32 here)
    np.testing.assert_allclose(oracle.softmax_f32(s + np.float32(8.0)), p, rtol=1e-5, atol=1e-12)
