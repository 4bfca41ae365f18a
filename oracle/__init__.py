"""CPU oracle of the NVFP4 hot path -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline`` leg
may import this package. It wraps the plain C reference ``nvfp4_oracle.c``
(brute-force rounding, FP64 accumulation) with numpy arrays and composes its
primitives into the three operations of the library:

* ``quantize`` / ``quantize_aug``  -- NVFP4 quantization, optionally with RMSNorm,
  channel gather and appended residue columns (ARCQuant article on zizhi168.cn,
  sections 3.1-3.2; ResServe abstract);
* ``gemm``                         -- y = S_a S_w deq(A) deq(W)^T in FP64;
* ``gemm_residue``                 -- the same product over X_aug and
  W_aug = [W' | W'[:, :S]] (ARCQuant article, section 3.1 formula and 3.2
  "unified GEMM" over K+S).

It shares no code with the HIP library. All inputs are host numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = C.CDLL(path)
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        i64 = C.c_int64
        vp = C.c_void_p
        L.or_e2m1_value.argtypes = [C.c_int]; L.or_e2m1_value.restype = C.c_double
        L.or_e4m3_value.argtypes = [C.c_int]; L.or_e4m3_value.restype = C.c_double
        L.or_e2m1_encode.argtypes = [C.c_float]; L.or_e2m1_encode.restype = C.c_int
        L.or_e4m3_encode.argtypes = [C.c_float]; L.or_e4m3_encode.restype = C.c_int
        L.or_tensor_scale.argtypes = [f32p, i64, i64, i64]; L.or_tensor_scale.restype = C.c_float
        L.or_quantize.argtypes = [f32p, i64, i64, i64, vp, u8p, i64, u8p, i64, vp]
        L.or_quantize.restype = i64
        L.or_dequantize.argtypes = [u8p, i64, u8p, i64, C.c_float, i64, i64, f64p, i64]
        L.or_dequantize_f32.argtypes = [u8p, i64, u8p, i64, C.c_float, i64, i64, f32p, i64]
        L.or_rmsnorm.argtypes = [f32p, i64, i64, i64, f32p, C.c_float, f32p, i64]
        L.or_channel_absmax.argtypes = [f32p, i64, i64, i64, vp, C.c_float, f32p]
        L.or_perm_from_absmax.argtypes = [f32p, i64, i32p]
        L.or_quantize_aug.argtypes = [f32p, i64, i64, i64, vp, C.c_float, vp, vp, i64, vp,
                                      u8p, i64, u8p, i64, vp]
        L.or_quantize_aug.restype = i64
        L.or_gemm.argtypes = [u8p, i64, u8p, i64, C.c_float, u8p, i64, u8p, i64, C.c_float,
                              i64, i64, i64, f64p, i64]
        L.or_gemm_pairs.argtypes = [u8p, i64, u8p, i64, C.c_float, u8p, i64, u8p, i64, C.c_float,
                                    i64, i64p, i64p, i64, f64p]
        L.or_gemm_exact.argtypes = [u8p, i64, u8p, i64, C.c_float, u8p, i64, u8p, i64, C.c_float,
                                    i64, i64, i64, f64p, i64]
        L.or_gemm_exact.restype = C.c_int
        L.or_e8m0_value.argtypes = [C.c_int]; L.or_e8m0_value.restype = C.c_double
        L.or_mx_block_exponent.argtypes = [f32p]; L.or_mx_block_exponent.restype = C.c_int
        L.or_mx_quantize.argtypes = [f32p, i64, i64, i64, u8p, i64, u8p, i64]
        L.or_mx_dequantize.argtypes = [u8p, i64, u8p, i64, i64, i64, f64p, i64]
        L.or_mx_quantize_aug.argtypes = [f32p, i64, i64, i64, i64, u8p, i64, u8p, i64]
        L.or_mx_gemm.argtypes = [u8p, i64, u8p, i64, u8p, i64, u8p, i64, i64, i64, i64, f64p, i64]
        _lib = L
    return _lib


def _f32(x) -> np.ndarray:
    """Accept numpy arrays or torch tensors (any float dtype; bf16 is exact in fp32)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


class QTensor:
    """An NVFP4 tensor in the canonical layout: codes [rows][K/2], scales [rows][K/16], S."""

    def __init__(self, codes: np.ndarray, scales: np.ndarray, S: float, K: int):
        self.codes, self.scales, self.S, self.K = codes, scales, np.float32(S), K
        self.near_midpoint = 0

    @property
    def rows(self) -> int:
        return self.codes.shape[0]


def e2m1_value(code: int) -> float:
    return lib().or_e2m1_value(code)


def e4m3_value(byte: int) -> float:
    return lib().or_e4m3_value(byte)


def e2m1_encode(q: float) -> int:
    return lib().or_e2m1_encode(float(np.float32(q)))


def e4m3_encode(v: float) -> int:
    return lib().or_e4m3_encode(float(np.float32(v)))


def tensor_scale(x) -> np.float32:
    x = _f32(x)
    rows, K = x.shape
    return np.float32(lib().or_tensor_scale(x, rows, K, K))


def _alloc(rows: int, K: int):
    return np.zeros((rows, K // 2), np.uint8), np.zeros((rows, K // 16), np.uint8)


def quantize(x, static_S=None) -> QTensor:
    x = _f32(x)
    rows, K = x.shape
    assert K % 16 == 0
    codes, scales = _alloc(rows, K)
    S = np.zeros(1, np.float32)
    sp = np.array([static_S], np.float32) if static_S is not None else None
    near = lib().or_quantize(x, rows, K, K, sp.ctypes.data if sp is not None else None,
                             codes, K // 2, scales, K // 16, S.ctypes.data)
    q = QTensor(codes, scales, S[0], K)
    q.near_midpoint = int(near)
    return q


def quantize_aug(x, gamma=None, eps: float = 1e-6, perm=None, S_cols: int = 0,
                 static_S=None, smooth=None) -> QTensor:
    """X_aug of the fused quantizer: RMSNorm (gamma), diagonal smoothing (per input
    channel), channel gather (perm), NVFP4 quantization and S_cols residue columns."""
    x = _f32(x)
    rows, K = x.shape
    Ka = K + S_cols
    assert K % 16 == 0 and S_cols % 16 == 0 and 0 <= S_cols <= K
    codes, scales = _alloc(rows, Ka)
    S = np.zeros(1, np.float32)
    g = _f32(gamma) if gamma is not None else None
    sm = _f32(smooth) if smooth is not None else None
    p = np.ascontiguousarray(perm, dtype=np.int32) if perm is not None else None
    sp = np.array([static_S], np.float32) if static_S is not None else None
    near = lib().or_quantize_aug(x, rows, K, K, g.ctypes.data if g is not None else None,
                                 np.float32(eps), sm.ctypes.data if sm is not None else None,
                                 p.ctypes.data if p is not None else None,
                                 S_cols, sp.ctypes.data if sp is not None else None,
                                 codes, Ka // 2, scales, Ka // 16, S.ctypes.data)
    q = QTensor(codes, scales, S[0], Ka)
    q.near_midpoint = int(near)
    return q


def dequantize(q: QTensor) -> np.ndarray:
    out = np.zeros((q.rows, q.K), np.float64)
    lib().or_dequantize(q.codes, q.codes.shape[1], q.scales, q.scales.shape[1], q.S,
                        q.rows, q.K, out, q.K)
    return out


def dequantize_f32(q: QTensor) -> np.ndarray:
    out = np.zeros((q.rows, q.K), np.float32)
    lib().or_dequantize_f32(q.codes, q.codes.shape[1], q.scales, q.scales.shape[1], q.S,
                            q.rows, q.K, out, q.K)
    return out


def rmsnorm(x, gamma, eps: float = 1e-6) -> np.ndarray:
    x = _f32(x)
    g = _f32(gamma)
    rows, K = x.shape
    y = np.zeros((rows, K), np.float32)
    lib().or_rmsnorm(x, rows, K, K, g, np.float32(eps), y, K)
    return y


def channel_absmax(x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    x = _f32(x)
    rows, K = x.shape
    g = _f32(gamma) if gamma is not None else None
    v = np.zeros(K, np.float32)
    lib().or_channel_absmax(x, rows, K, K, g.ctypes.data if g is not None else None,
                            np.float32(eps), v)
    return v


def perm_from_absmax(v) -> np.ndarray:
    v = _f32(v)
    perm = np.zeros(v.shape[0], np.int32)
    lib().or_perm_from_absmax(v, v.shape[0], perm)
    return perm


def calibrate_perm(x_cal, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """Channel order for the outlier reorder: descending calibration absmax."""
    return perm_from_absmax(channel_absmax(x_cal, gamma, eps))


def gemm(a: QTensor, w: QTensor) -> np.ndarray:
    assert a.K == w.K
    M, N, K = a.rows, w.rows, a.K
    y = np.zeros((M, N), np.float64)
    lib().or_gemm(a.codes, a.codes.shape[1], a.scales, a.scales.shape[1], a.S,
                  w.codes, w.codes.shape[1], w.scales, w.scales.shape[1], w.S, M, N, K, y, N)
    return y


def dequantize_unscaled(q: QTensor) -> np.ndarray:
    """e(c) * d in FP64 (exact), without the tensor scale."""
    return dequantize(QTensor(q.codes, q.scales, 1.0, q.K))


def gemm_blas(a: QTensor, w: QTensor) -> np.ndarray:
    """The product of ``gemm`` with numpy's float64 matmul as its summation step,
    for references at full workload sizes. Every e(c)d is an integer multiple of
    2^-10 and every product of two a multiple of 2^-20; while the partial sums stay
    below 2^33 in magnitude (as on every workload here) each of them is exact in
    FP64 in any order, so this equals ``gemm`` bit for bit (a test pins that)."""
    assert a.K == w.K
    y = dequantize_unscaled(a) @ dequantize_unscaled(w).T
    return y * (np.float64(a.S) * np.float64(w.S))


def gemm_pairs(a: QTensor, w: QTensor, ms, ns) -> np.ndarray:
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    y = np.zeros(ms.shape[0], np.float64)
    lib().or_gemm_pairs(a.codes, a.codes.shape[1], a.scales, a.scales.shape[1], a.S,
                        w.codes, w.codes.shape[1], w.scales, w.scales.shape[1], w.S,
                        a.K, ms, ns, ms.shape[0], y)
    return y


def gemm_exact(a: QTensor, w: QTensor) -> np.ndarray:
    M, N, K = a.rows, w.rows, a.K
    y = np.zeros((M, N), np.float64)
    rc = lib().or_gemm_exact(a.codes, a.codes.shape[1], a.scales, a.scales.shape[1], a.S,
                             w.codes, w.codes.shape[1], w.scales, w.scales.shape[1], w.S,
                             M, N, K, y, N)
    if rc != 0:
        raise OverflowError("exact accumulation out of range")
    return y


def weight_aug(w_perm, S_cols: int) -> QTensor:
    """W_aug = [W' | W'[:, :S]] quantized as one tensor (W' already in channel order)."""
    w = _f32(w_perm)
    if S_cols:
        w = np.ascontiguousarray(np.concatenate([w, w[:, :S_cols]], axis=1))
    return quantize(w)


def gemm_residue(x, w_perm, S_cols: int, gamma=None, eps: float = 1e-6, perm=None):
    """Y = s_aug [Q(X') | Q(R)] [Q(W') | Q(W'_o)]^T; returns (y, X_aug, W_aug)."""
    xa = quantize_aug(x, gamma, eps, perm, S_cols)
    wa = weight_aug(w_perm, S_cols)
    return gemm(xa, wa), xa, wa


def gemm_error(y, y_ref) -> float:
    """Max |y - y*| / max(|y*|, 1e-3 max|y*|): relative error floored near zero."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return 0.0
    floor = 1e-3 * np.max(np.abs(y_ref))
    den = np.maximum(np.abs(y_ref), floor if floor > 0 else 1e-30)
    return float(np.max(np.abs(y - y_ref) / den))


# ---------------------------------------------------------------------- MXFP4
# E2M1 codes (the same packing) with one E8M0 scale byte per 32 elements along K
# and no tensor scale; the rule is stated in nvfp4_oracle.c.

class MXTensor:
    """An MXFP4 tensor in the canonical layout: codes [rows][K/2], scales [rows][K/32]."""

    def __init__(self, codes: np.ndarray, scales: np.ndarray, K: int):
        self.codes, self.scales, self.K = codes, scales, K

    @property
    def rows(self) -> int:
        return self.codes.shape[0]


def e8m0_value(byte: int) -> float:
    return lib().or_e8m0_value(byte)


def mx_block_exponent(v32) -> int:
    v = np.ascontiguousarray(v32, dtype=np.float32)
    assert v.shape == (32,)
    return int(lib().or_mx_block_exponent(v))


def mx_quantize(x, S_cols: int = 0) -> MXTensor:
    """MXFP4 quantization of x (rows x K, K % 32 == 0); with S_cols > 0, X_aug = [Q(x) | Q(R)]
    with R = x - deq(Q(x)) on columns [0, S_cols)."""
    x = _f32(x)
    rows, K = x.shape
    assert K % 32 == 0 and S_cols % 32 == 0 and 0 <= S_cols <= K
    Ka = K + S_cols
    codes, scales = np.zeros((rows, Ka // 2), np.uint8), np.zeros((rows, Ka // 32), np.uint8)
    if S_cols:
        lib().or_mx_quantize_aug(x, rows, K, K, S_cols, codes, Ka // 2, scales, Ka // 32)
    else:
        lib().or_mx_quantize(x, rows, K, K, codes, K // 2, scales, K // 32)
    return MXTensor(codes, scales, Ka)


def mx_dequantize(q: MXTensor) -> np.ndarray:
    out = np.zeros((q.rows, q.K), np.float64)
    lib().or_mx_dequantize(q.codes, q.codes.shape[1], q.scales, q.scales.shape[1], q.rows, q.K, out, q.K)
    return out


def mx_gemm(a: MXTensor, w: MXTensor) -> np.ndarray:
    assert a.K == w.K
    y = np.zeros((a.rows, w.rows), np.float64)
    lib().or_mx_gemm(a.codes, a.codes.shape[1], a.scales, a.scales.shape[1],
                     w.codes, w.codes.shape[1], w.scales, w.scales.shape[1], a.rows, w.rows, a.K, y, w.rows)
    return y


def mx_gemm_blas(a: MXTensor, w: MXTensor) -> np.ndarray:
    """mx_gemm with numpy's float64 matmul as the summation step (sums in another order),
    for references at full workload sizes; a test bounds its distance to mx_gemm."""
    assert a.K == w.K
    return mx_dequantize(a) @ mx_dequantize(w).T


def mx_weight_aug(w: MXTensor, S_cols: int) -> MXTensor:
    """W_aug = [W | W[:, :S]] of an MXFP4 weight: the tail repeats the head's first S
    columns (their codes and block scales)."""
    return MXTensor(np.ascontiguousarray(np.concatenate([w.codes, w.codes[:, :S_cols // 2]], axis=1)),
                    np.ascontiguousarray(np.concatenate([w.scales, w.scales[:, :S_cols // 32]], axis=1)),
                    w.K + S_cols)



# ------------------------------------------------- decode attention (compensated)
# ResServe abstract: the FP4 activation base plus FP4-quantized residue is applied
# "to linear layers and decode attention". Reading (the pages give no attention
# formula; this is scaled dot-product attention for one decode query per head):
# the KV cache is stored in NVFP4 like a weight -- K as [H*T, D] (row h*T + t,
# blocks along D), V transposed as [H*D, T] (row h*D + j, blocks along T), one
# tensor scale each -- and the two activation operands of the step, the query
# q_h and the probabilities p_h, carry the base + residue of the linear layers:
#   s_h = ( [Q(q_h) | Q(R_q)] . [K_h | K_h]^T ) / sqrt(D)       (the residue product)
#   p_h = softmax(s_h)                  in FP32: m = max s, e = exp(s - m), p = e / sum(e)
#   o_h =   [Q(p_h) | Q(R_p)] . [Vt_h | Vt_h]^T
# with each q_h and p_h quantized as its own tensor (its own tensor scale), and
# compensate=False dropping the residue columns. Products are FP64 (gemm).

def _rows(q: QTensor, r0: int, r1: int, dup: bool) -> QTensor:
    """Rows [r0, r1) of a quantized tensor, with its codes and scales repeated once
    along K when dup (W_aug = [W | W]: the tail is W's own columns)."""
    c, s = q.codes[r0:r1, : q.K // 2], q.scales[r0:r1, : q.K // 16]
    if dup:
        c, s = np.concatenate([c, c], axis=1), np.concatenate([s, s], axis=1)
    return QTensor(np.ascontiguousarray(c), np.ascontiguousarray(s), q.S, q.K * (2 if dup else 1))


def softmax_f32(s) -> np.ndarray:
    """p = e / sum(e), e = exp(s - max s), every step in FP32 (numpy float32 ops)."""
    s = np.asarray(s, np.float32)
    e = np.exp(s - np.max(s)).astype(np.float32)
    return (e / np.float32(np.sum(e, dtype=np.float32))).astype(np.float32)


def decode_attention(q, k_cache: QTensor, vt_cache: QTensor, H: int, T: int, D: int,
                     compensate: bool = True, return_p: bool = False):
    """o [H, D] (FP64) of the compensated decode attention above; q is [H, D]."""
    q = _f32(q)
    assert q.shape == (H, D) and k_cache.K == D and k_cache.rows == H * T
    assert vt_cache.K == T and vt_cache.rows == H * D and D % 16 == 0 and T % 16 == 0
    o = np.zeros((H, D), np.float64)
    ps = np.zeros((H, T), np.float32)
    inv = 1.0 / np.sqrt(np.float64(D))
    for h in range(H):
        qa = quantize_aug(q[h:h + 1], S_cols=D if compensate else 0)
        y = gemm(qa, _rows(k_cache, h * T, (h + 1) * T, compensate))[0]
        p = softmax_f32((y * inv).astype(np.float32))
        ps[h] = p
        pa = quantize_aug(p[None, :], S_cols=T if compensate else 0)
        o[h] = gemm(pa, _rows(vt_cache, h * D, (h + 1) * D, compensate))[0]
    return (o, ps) if return_p else o
