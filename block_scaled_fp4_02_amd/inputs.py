"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

This module only draws random tensors; it holds none of the NVFP4 arithmetic.
Every tensor comes from its own numpy stream ``default_rng([0, cfg, sub, tensor])``
so that shapes never interact:

* activations ``X``: standard normal, with a fixed set of outlier channels
  (the same columns in every row) multiplied by a constant before the cast;
* weights ``W``: normal with the stated sigma;
* RMSNorm weight ``gamma``: uniform(0.5, 1.5);
* calibration rows ``X_cal``: the activation law on a separate stream.

All float tensors are rounded to bfloat16 (round-to-nearest-even, by torch on
the CPU) and returned as ``torch.bfloat16`` CPU tensors.

The shapes and laws stand in for the linear layers of the Llama-3.1-8B
(4096 / 14336 / 6144) and Llama-3.3-70B (8192 / 28672) models that the pages
evaluate; no model weights, calibration sets or benchmark items are used.
"""
from __future__ import annotations

import numpy as np
import torch

# tensor ids inside a config's seed sequence
T_X, T_W, T_OUTLIER, T_GAMMA, T_XCAL = 1, 2, 3, 4, 5

# decode GEMM sweep shapes (K, N)
DECODE_SHAPES = [(4096, 14336), (14336, 4096), (4096, 6144)]
DECODE_MS = [1, 2, 4, 8, 16]
PREFILL_SHAPES = [(8192, 28672), (28672, 8192)]
PREFILL_MS = [512, 2048, 8192]
RESIDUE_MS = [1, 8, 16]
AUG_S = [128, 256, 512]


def _rng(cfg: int, sub: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([0, cfg, sub, tensor])


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def outlier_columns(cfg: int, sub: int, K: int, frac: float) -> np.ndarray:
    """The fixed outlier channel indices: round(frac*K) columns without replacement."""
    n_out = int(round(frac * K))
    return np.sort(_rng(cfg, sub, T_OUTLIER).choice(K, n_out, replace=False))


def activations(cfg: int, sub: int, rows: int, K: int, frac: float, mult: float,
                tensor: int = T_X) -> torch.Tensor:
    """N(0,1) activations with ``round(frac*K)`` outlier channels scaled by ``mult``."""
    x = _rng(cfg, sub, tensor).standard_normal((rows, K), dtype=np.float32)
    cols = outlier_columns(cfg, sub, K, frac)
    x[:, cols] *= np.float32(mult)
    return _bf16(x)


def weights(cfg: int, sub: int, N: int, K: int, sigma: float) -> torch.Tensor:
    w = _rng(cfg, sub, T_W).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return _bf16(w)


def gamma(cfg: int, sub: int, K: int) -> torch.Tensor:
    g = _rng(cfg, sub, T_GAMMA).uniform(0.5, 1.5, size=K).astype(np.float32)
    return _bf16(g)


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def gemv_4096(seed_cfg: int = 1):
    """Single W4A4 GEMV: x[1x4096] (1% channels x50), W[4096x4096] ~ N(0, 0.02)."""
    x = activations(seed_cfg, 0, 1, 4096, 0.01, 50.0)
    w = weights(seed_cfg, 0, 4096, 4096, 0.02)
    return x, w


def decode_sweep(shape_idx: int, m_max: int = 16):
    """Small-M decode GEMM: X[m_max x K] (1% x50) and W[N x K] ~ N(0, 0.02).

    The sweep over M uses the first M rows of X."""
    K, N = DECODE_SHAPES[shape_idx]
    x = activations(2, shape_idx, m_max, K, 0.01, 50.0)
    w = weights(2, shape_idx, N, K, 0.02)
    return x, w


def residue_8192(m_max: int = 16):
    """Residue-compensated GEMM: X[m_max x 8192] (2% x100), W[8192 x 8192] ~ N(0, 0.02)."""
    x = activations(3, 0, m_max, 8192, 0.02, 100.0)
    w = weights(3, 0, 8192, 8192, 0.02)
    return x, w


def outlier_aug(rows: int = 64, K: int = 4096, N: int = 14336, cal_rows: int = 512):
    """Augmented-channel GEMM: X[64 x 4096] (1% x50), gamma ~ U(0.5,1.5),
    X_cal[512 x 4096] with the same law (separate stream), W[14336 x 4096] ~ N(0, 0.02)."""
    x = activations(4, 0, rows, K, 0.01, 50.0)
    g = gamma(4, 0, K)
    xcal = activations(4, 0, cal_rows, K, 0.01, 50.0, tensor=T_XCAL)
    w = weights(4, 0, N, K, 0.02)
    return x, g, xcal, w


def prefill(shape_idx: int, M: int):
    """Prefill GEMM: X[M x K] (1% x50), W[N x K] ~ N(0, 0.015)."""
    K, N = PREFILL_SHAPES[shape_idx]
    x = activations(5, shape_idx, M, K, 0.01, 50.0)
    w = weights(5, shape_idx, N, K, 0.015)
    return x, w


def small_random(seed: int, rows: int, K: int, scale: float = 1.0, outlier_frac: float = 0.02,
                 mult: float = 40.0) -> torch.Tensor:
    """Small seeded tensors for parity cases (ragged shapes, several tiles)."""
    x = np.random.default_rng([0, 100, seed]).standard_normal((rows, K), dtype=np.float32) * np.float32(scale)
    if outlier_frac > 0 and K > 0:
        cols = np.random.default_rng([0, 101, seed]).choice(K, max(1, int(round(outlier_frac * K))), replace=False)
        x[:, cols] *= np.float32(mult)
    return _bf16(x)


# decode attention: 32 heads of dimension 128 over 4096 cached tokens (the
# Llama-3.1-8B query geometry, one KV head per query head)
ATTN_SHAPE = (32, 4096, 128)


def attention(H: int, T: int, D: int, sub: int = 0):
    """Decode attention inputs (config 6 streams): q [H x D], K [H*T x D] (row h*T + t)
    and V transposed, Vt [H*D x T] (row h*D + j), all N(0, 1) in bf16; the query has
    1% outlier channels x 50 like the other activations."""
    q = activations(6, sub, H, D, 0.01, 50.0)
    k = _bf16(_rng(6, sub, T_W).standard_normal((H * T, D), dtype=np.float32))
    v = _rng(6, sub, T_XCAL).standard_normal((H, T, D), dtype=np.float32)
    vt = _bf16(np.ascontiguousarray(v.transpose(0, 2, 1)).reshape(H * D, T))
    return q, k, vt
