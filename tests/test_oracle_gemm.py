"""Pins of the oracle's W4A4 product (ARCQuant article, section 3.1 formula).

* FP64 accumulation equals an exact integer accumulation bit for bit (every
  product is an integer multiple of 2^-20, so the FP64 sums are exact);
* it equals numpy's float64 matmul of the dequantized operands (a library
  routine) to within rounding;
* brute force over a single 16-element block, one-hot weight rows, zero weights;
* the augmented-K identity Y = Q(X)Q(W)^T + Q(R)Q(W_o)^T = s_aug [QX|QR][QW|QWo]^T,
  and that a whole-block channel permutation applied to both operands leaves
  the product unchanged;
* the residue lowers the activation-side product error, as the ResServe
  abstract states for compensated kernels.
"""
import itertools

import numpy as np
import pytest

from block_scaled_fp4_02_amd import inputs


def test_gemm_fp64_equals_exact_and_numpy(orc):
    x = inputs.small_random(1, 5, 256)
    w = inputs.small_random(2, 37, 256, scale=0.02)
    a, b = orc.quantize(x), orc.quantize(w)
    y = orc.gemm(a, b)
    ye = orc.gemm_exact(a, b)
    assert np.array_equal(y, ye)
    ref = (orc.dequantize(a) @ orc.dequantize(b).T)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_gemm_blas_equals_gemm(orc):
    """The library-matmul form used for full-size references is the same product,
    bit for bit (all partial sums exact), on a decode-sweep-shaped slice."""
    x, w = inputs.decode_sweep(1)
    a, b = orc.quantize(x[:, :2048]), orc.quantize(w[:300, :2048])
    assert np.array_equal(orc.gemm_blas(a, b), orc.gemm(a, b))
    a = orc.quantize(inputs.small_random(7, 9, 528))
    b = orc.quantize(inputs.small_random(8, 77, 528, scale=0.02))
    assert np.array_equal(orc.gemm_blas(a, b), orc.gemm(a, b))


def test_gemm_workload_exact(orc):
    x, w = inputs.gemv_4096()
    a, b = orc.quantize(x), orc.quantize(w[:512])
    assert np.array_equal(orc.gemm(a, b), orc.gemm_exact(a, b))


def test_gemm_single_block_brute_force(orc):
    x = inputs.small_random(3, 2, 16)
    w = inputs.small_random(4, 3, 16)
    a, b = orc.quantize(x), orc.quantize(w)
    da, dw = orc.dequantize(a), orc.dequantize(b)
    y = orc.gemm(a, b)
    for m, n in itertools.product(range(2), range(3)):
        s = 0.0
        for k in range(16):
            s += float(da[m, k]) * float(dw[n, k])
        assert abs(y[m, n] - s) <= 1e-12 * max(1.0, abs(s))


def test_gemm_one_hot_and_zero(orc):
    x = inputs.small_random(5, 3, 64)
    a = orc.quantize(x)
    da = orc.dequantize(a)
    # one-hot W rows holding v = 2688 * 2^-12, so S_w = 2^-12 exactly and deq(w) = v
    N, v = 64, np.float32(2688 * 2.0 ** -12)
    w = np.zeros((N, 64), np.float32)
    w[np.arange(N), np.arange(N)] = v
    b = orc.quantize(w)
    assert b.S == np.float32(2.0 ** -12)
    dw = orc.dequantize(b)
    assert np.all(dw[np.arange(N), np.arange(N)] == v)
    assert np.array_equal(orc.gemm(a, b), da * np.float64(v))
    z = orc.quantize(np.zeros((4, 64), np.float32))
    assert not orc.gemm(a, z).any()


def test_gemm_pairs_matches_full(orc):
    x = inputs.small_random(6, 7, 128)
    w = inputs.small_random(7, 19, 128, scale=0.02)
    a, b = orc.quantize(x), orc.quantize(w)
    y = orc.gemm(a, b)
    ms = np.array([0, 6, 3, 3]); ns = np.array([18, 0, 7, 8])
    assert np.array_equal(orc.gemm_pairs(a, b, ms, ns), y[ms, ns])


def test_block_permutation_invariance(orc):
    x = inputs.small_random(8, 4, 128)
    w = inputs.small_random(9, 9, 128, scale=0.02)
    a, b = orc.quantize(x), orc.quantize(w)
    blocks = np.random.default_rng(2).permutation(8)
    perm = (blocks[:, None] * 16 + np.arange(16)[None, :]).reshape(-1).astype(np.int32)
    ap = orc.quantize_aug(x, perm=perm)
    bp = orc.quantize_aug(w, perm=perm)
    assert np.array_equal(orc.gemm(a, b), orc.gemm(ap, bp))


def test_augmented_identity(orc):
    x, w = inputs.residue_8192(4)
    K = 8192
    w = w[:64]
    for S in [0, 128, K]:
        y, xa, wa = orc.gemm_residue(x, w, S)
        qx, qw = orc.quantize(x), orc.quantize(w)
        assert xa.S == qx.S and wa.S == qw.S
        # W_aug tail == head (never materialised by the kernels)
        assert np.array_equal(wa.codes[:, K // 2:], qw.codes[:, :S // 2])
        assert np.array_equal(wa.scales[:, K // 16:], qw.scales[:, :S // 16])
        base = orc.gemm(qx, qw)
        if S == 0:
            assert np.array_equal(y, base)
            continue
        # Y = Q(X)Q(W)^T + Q(R)Q(W_o)^T
        R = orc.QTensor(np.ascontiguousarray(xa.codes[:, K // 2:]), np.ascontiguousarray(xa.scales[:, K // 16:]), xa.S, S)
        Wo = orc.QTensor(np.ascontiguousarray(qw.codes[:, :S // 2]), np.ascontiguousarray(qw.scales[:, :S // 16]), qw.S, S)
        assert np.allclose(y, base + orc.gemm(R, Wo), rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_residue_improves_precision(orc):
    x, w = inputs.residue_8192(8)
    w = w[:256]
    xf = x.float().numpy().astype(np.float64)
    qw = orc.quantize(w)
    ref = xf @ orc.dequantize(qw).T
    y_base = orc.gemm(orc.quantize(x), qw)
    y_res, _, _ = orc.gemm_residue(x, w, 8192)
    r = np.linalg.norm(y_res - ref) / np.linalg.norm(y_base - ref)
    assert r <= 0.25, r


def test_gemm_error_metric(orc):
    y_ref = np.array([[1.0, -2.0, 1e-9, 0.0]])
    assert orc.gemm_error(y_ref, y_ref) == 0.0
    y = y_ref.copy(); y[0, 1] += 2e-3 * 2.0
    assert abs(orc.gemm_error(y, y_ref) - 2e-3) < 1e-12
    y = y_ref.copy(); y[0, 2] += 1e-6          # floored at 1e-3 * max = 2e-3
    assert abs(orc.gemm_error(y, y_ref) - 5e-4) < 1e-9
