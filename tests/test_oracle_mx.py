"""Pins of the oracle's MXFP4 functions (E2M1 elements, one E8M0 power-of-two scale per
32 elements along K; the 32-element blocks and E8M0 scales of the MX formats in the
ARCQuant article, sections 2.2 and 4.2, and MXFP4 as named in the ResServe abstract).

The scale rule is pinned by its characterisation rather than by its formula: the
chosen 2^e is the one power of two with 4 <= amax / 2^e < 8 (so the block maximum
lands on E2M1's top binade and saturates at most to 6), clamped to E8M0's range.
Also: E8M0 values against torch's float8_e8m0fnu decoder, exact reconstruction of
on-grid inputs, brute-force nearest-code rounding, the per-element error bound, the
residue columns written out in numpy, and the product against numpy's float64 matmul.
"""
import json
import os

import numpy as np
import pytest

from block_scaled_fp4_02_amd import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_format.json")))
BOOK = np.array(GOLD["e2m1_codebook"]["value"])


def unpack(codes):
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


def values(c):
    v = BOOK[c & 7]
    return np.where(c & 8, -v, v)


def test_e8m0_table(orc):
    import torch
    b = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)
    got = np.array([orc.e8m0_value(int(v)) for v in b])
    assert np.array_equal(got[1:], ref[1:])            # torch's decoder treats byte 0 as 2^-127 too
    assert got[0] == 2.0 ** -127 and got[127] == 1.0 and got[254] == 2.0 ** 127
    assert np.isnan(orc.e8m0_value(255))


def test_scale_characterisation(orc):
    rng = np.random.default_rng(1)
    for t in range(400):
        v = rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** rng.integers(-110, 110))
        e = orc.mx_block_exponent(v)
        amax = float(np.abs(v).max())
        assert 4.0 <= amax / 2.0 ** e < 8.0, (t, e, amax)
    # clamping at both ends of E8M0, and the all-zero block
    assert orc.mx_block_exponent(np.full(32, 2.0 ** -140, np.float32)) == -127
    assert orc.mx_block_exponent(np.full(32, 3.0e38, np.float32)) == 127 - 2
    assert orc.mx_block_exponent(np.zeros(32, np.float32)) == -127


def test_grid_inputs_reconstruct_exactly(orc):
    rng = np.random.default_rng(2)
    rows, K = 5, 512
    nb = K // 32
    codes = rng.integers(0, 16, size=(rows, K))
    codes[:, ::32] = np.where(rng.random((rows, nb)) < 0.5, 6, 15)     # |e| = 4 or 6 in every block
    E = rng.integers(-60, 60, size=(rows, nb))
    x = (values(codes) * np.repeat(2.0 ** E, 32, axis=1)).astype(np.float32)
    q = orc.mx_quantize(x)
    assert np.array_equal(q.scales.astype(np.int64), E + 127)
    assert np.array_equal(orc.mx_dequantize(q), x.astype(np.float64))
    # the same codes (+0 and -0 both decode to 0: compare magnitudes where the value is zero)
    got = unpack(q.codes)
    nz = values(codes) != 0
    assert np.array_equal(got[nz], codes[nz]) and np.all((got[~nz] & 7) == 0)


def test_brute_force_rounding_and_error_bound(orc):
    x = inputs.small_random(3, 8, 1024).float().numpy()
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    q = orc.mx_quantize(x)
    c = unpack(q.codes)
    e = q.scales.astype(np.int64) - 127
    s = np.repeat(2.0 ** e, 32, axis=1)
    qv = x.astype(np.float64) / s
    # nearest E2M1 magnitude by brute force, ties to the even code, saturating at 6
    dist = np.abs(np.abs(qv)[..., None] - BOOK[None, None, :])
    best = np.argmin(dist + (np.arange(8) & 1) * 1e-12, axis=-1)
    best = np.where(np.abs(qv) >= 6.0, 7, best)
    assert np.array_equal(c & 7, best)
    assert np.array_equal((c >> 3) == 1, np.signbit(x))
    deq = orc.mx_dequantize(q)
    a = np.abs(qv)
    h = np.where(a <= 2, 0.25, np.where(a <= 4, 0.5, np.where(a <= 6, 1.0, a - 6.0)))
    assert np.all(np.abs(x - deq) <= s * h * (1 + 2.0 ** -40))
    assert np.all(q.scales[0:2, 0] == 0) and np.all(deq[0:2, :32] == 0)


def test_residue_tail_from_numpy(orc):
    x = inputs.small_random(4, 6, 1024).float().numpy()
    S = 256
    xa = orc.mx_quantize(x, S_cols=S)
    q = orc.mx_quantize(x)
    assert np.array_equal(xa.codes[:, :512], q.codes) and np.array_equal(xa.scales[:, :32], q.scales)
    deq = (values(unpack(q.codes)) * np.repeat(2.0 ** (q.scales.astype(np.int64) - 127), 32, axis=1)).astype(np.float32)
    R = (x[:, :S] - deq[:, :S]).astype(np.float32)
    qr = orc.mx_quantize(np.ascontiguousarray(R))
    assert np.array_equal(xa.codes[:, 512:], qr.codes) and np.array_equal(xa.scales[:, 32:], qr.scales)
    # two stages leave less error than one on every block
    d = orc.mx_dequantize(xa)
    e1 = np.abs(x[:, :S] - d[:, :S]).reshape(6, -1, 32).max(axis=2)
    e2 = np.abs(x[:, :S] - d[:, :S] - d[:, 1024:]).reshape(6, -1, 32).max(axis=2)
    assert np.all(e2 <= e1) and e2.sum() < 0.5 * e1.sum()


def test_gemm_against_numpy_and_brute_force(orc):
    a = orc.mx_quantize(inputs.small_random(5, 7, 512))
    w = orc.mx_quantize(inputs.small_random(6, 33, 512, scale=0.02))
    y = orc.mx_gemm(a, w)
    ref = orc.mx_dequantize(a) @ orc.mx_dequantize(w).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(orc.mx_gemm_blas(a, w), ref)
    da, dw = orc.mx_dequantize(a), orc.mx_dequantize(w)
    for m, n in [(0, 0), (6, 32), (3, 17)]:
        s = 0.0
        for k in range(512):
            s += float(da[m, k]) * float(dw[n, k])
        assert abs(y[m, n] - s) <= 1e-12 * max(1.0, abs(s))


def test_augmented_identity(orc):
    """Y over X_aug and W_aug = [W | W[:, :S]] equals Q(X) Q(W)^T + Q(R) Q(W[:, :S])^T."""
    x = inputs.small_random(7, 5, 512)
    w = orc.mx_quantize(inputs.small_random(8, 40, 512, scale=0.02))
    S = 128
    xa = orc.mx_quantize(x, S_cols=S)
    y = orc.mx_gemm(xa, orc.mx_weight_aug(w, S))
    d = orc.mx_dequantize(xa)
    ref = d[:, :512] @ orc.mx_dequantize(w).T + d[:, 512:] @ orc.mx_dequantize(w)[:, :S].T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
