"""Thin ctypes binding of libnvfp4 (include/nvfp4.h) for torch tensors.

Argument marshalling only: every step of the computation runs in the HIP
library. Loading fails loudly when ``libnvfp4.so`` is missing; there is no
fallback path. Device memory (outputs, workspace) comes from torch, and every
call is enqueued on torch's current HIP stream.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

BF16, FP32 = 0, 1
_STATUS = {0: "ok", 1: "null pointer", 2: "bad shape", 3: "misaligned", 4: "bad dtype",
           5: "workspace too small", 6: "unsupported", 7: "HIP error"}


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({_STATUS.get(status, '?')})")


ROWMAJOR, TILED = 0, 1


class _CTensor(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("ld_codes", C.c_int64), ("scales", C.c_void_p),
                ("ld_scales", C.c_int64), ("tensor_scale", C.c_void_p), ("rows", C.c_int64),
                ("K", C.c_int64), ("layout", C.c_int32)]


class _COpts(C.Structure):
    _fields_ = [("gamma", C.c_void_p), ("eps", C.c_float), ("perm", C.c_void_p),
                ("residue_cols", C.c_int64), ("static_tensor_scale", C.c_void_p), ("smooth", C.c_void_p)]


_lib = None
_lock = threading.Lock()

EXPORTS = ["nvfp4_quantize", "nvfp4_gemm", "nvfp4_gemm_noalloc", "nvfp4_gemm_residue", "nvfp4_mx_quantize",
           "nvfp4_mx_gemm", "nvfp4_mx_pack_tiled", "nvfp4_decode_attention", "nvfp4_pack_tiled", "nvfp4_channel_absmax",
           "nvfp4_perm_from_absmax", "nvfp4_workspace_size", "nvfp4_status_string",
           "nvfp4_last_error", "nvfp4_version", "nvfp4_host_e4m3_encode", "nvfp4_host_e2m1_encode"]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
            L = C.CDLL(LIB_PATH)
            vp, i64, sz = C.c_void_p, C.c_int64, C.c_size_t
            L.nvfp4_quantize.argtypes = [vp, C.c_int, i64, i64, i64, vp, vp, vp, sz, vp]
            L.nvfp4_gemm.argtypes = [vp, vp, C.c_int, i64, i64, i64, vp, vp, C.c_int, i64, vp, sz, vp]
            L.nvfp4_gemm_noalloc.argtypes = [vp, vp, C.c_int, i64, i64, i64, vp, vp, C.c_int, i64, vp]
            L.nvfp4_gemm_residue.argtypes = [vp, C.c_int, i64, i64, i64, vp, vp, vp, C.c_int, i64, vp,
                                             vp, sz, vp]
            L.nvfp4_pack_tiled.argtypes = [vp, vp, vp]
            L.nvfp4_mx_quantize.argtypes = [vp, C.c_int, i64, i64, i64, i64, vp, vp]
            L.nvfp4_mx_gemm.argtypes = [vp, vp, i64, vp, C.c_int, i64, vp, sz, vp]
            L.nvfp4_mx_pack_tiled.argtypes = [vp, vp, vp]
            L.nvfp4_decode_attention.argtypes = [vp, C.c_int, i64, i64, i64, vp, vp, i64, C.c_int, vp, i64,
                                                 vp, sz, vp]
            L.nvfp4_channel_absmax.argtypes = [vp, C.c_int, i64, i64, i64, vp, C.c_float, vp, vp, sz, vp]
            L.nvfp4_perm_from_absmax.argtypes = [vp, i64, vp]
            L.nvfp4_workspace_size.argtypes = [C.c_int, i64, i64, i64, i64]
            L.nvfp4_workspace_size.restype = sz
            L.nvfp4_status_string.argtypes = [C.c_int]
            L.nvfp4_status_string.restype = C.c_char_p
            L.nvfp4_last_error.restype = C.c_char_p
            L.nvfp4_host_e4m3_encode.argtypes = [C.c_float]
            L.nvfp4_host_e2m1_encode.argtypes = [C.c_float]
            for name in ("nvfp4_quantize", "nvfp4_gemm", "nvfp4_gemm_noalloc", "nvfp4_gemm_residue", "nvfp4_pack_tiled",
                         "nvfp4_mx_quantize", "nvfp4_mx_gemm", "nvfp4_mx_pack_tiled", "nvfp4_decode_attention",
                         "nvfp4_channel_absmax", "nvfp4_perm_from_absmax"):
                getattr(L, name).restype = C.c_int
            _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = lib().nvfp4_last_error().decode() if status == 7 else ""
        err = NVFP4Error(status, what + (f" [{msg}]" if msg else ""))
        raise err


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


class NVFP4Tensor:
    """Device NVFP4 tensor: codes u8, scales u8, scale [1] f32, in one of two layouts.

    Row-major: codes [rows, ld_codes], scales [rows, ld_scales]. Tiled (weights
    for the products): codes [ceil(rows/16), KU*4096], scales [ceil(rows/16),
    KU*512], KU = ceil(K/512), as documented in include/nvfp4.h."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, scale: torch.Tensor, K: int,
                 layout: int = ROWMAJOR, rows: int | None = None):
        self.codes, self.scales, self.scale, self.K, self.layout = codes, scales, scale, K, layout
        self._rows = codes.shape[0] if rows is None else rows

    @staticmethod
    def empty(rows: int, K: int, device="cuda") -> "NVFP4Tensor":
        ldc, lds = _round_up(max(K // 2, 1), 16), _round_up(max(K // 16, 1), 8)
        codes = torch.empty((rows, ldc), dtype=torch.uint8, device=device)
        scales = torch.empty((rows, lds), dtype=torch.uint8, device=device)
        scale = torch.empty((1,), dtype=torch.float32, device=device)
        return NVFP4Tensor(codes, scales, scale, K)

    @staticmethod
    def empty_tiled(rows: int, K: int, device="cuda") -> "NVFP4Tensor":
        nt, ku = (rows + 15) // 16, (K + 511) // 512
        codes = torch.empty((nt, ku * 4096), dtype=torch.uint8, device=device)
        scales = torch.empty((nt, ku * 512), dtype=torch.uint8, device=device)
        scale = torch.empty((1,), dtype=torch.float32, device=device)
        return NVFP4Tensor(codes, scales, scale, K, TILED, rows)

    @property
    def rows(self) -> int:
        return self._rows

    def clone(self) -> "NVFP4Tensor":
        return NVFP4Tensor(self.codes.clone(), self.scales.clone(), self.scale.clone(), self.K, self.layout,
                           self._rows)

    def c(self) -> _CTensor:
        ldc = self.codes.stride(0) if self.codes.dim() == 2 else 0
        lds = self.scales.stride(0) if self.scales.dim() == 2 else 0
        return _CTensor(self.codes.data_ptr(), ldc, self.scales.data_ptr(), lds, self.scale.data_ptr(),
                        self.rows, self.K, self.layout)

    def host(self):
        """(codes [rows, K/2], scales [rows, K/16], S) as numpy arrays on the host (row-major only)."""
        if self.layout != ROWMAJOR:
            raise ValueError("host() reads row-major tensors")
        return (self.codes[:, : self.K // 2].cpu().numpy(), self.scales[:, : self.K // 16].cpu().numpy(),
                self.scale.cpu().numpy()[0])


def pack_tiled(w: NVFP4Tensor) -> NVFP4Tensor:
    """The tiled copy of a row-major weight (nvfp4_pack_tiled), on the current stream."""
    out = NVFP4Tensor.empty_tiled(w.rows, w.K, device=w.codes.device)
    src, dst = w.c(), out.c()
    _check(lib().nvfp4_pack_tiled(C.byref(src), C.byref(dst), _stream()), "nvfp4_pack_tiled")
    return out


_ws = {}
_ws_retired = []


def workspace(nbytes: int, device) -> torch.Tensor:
    """A per-(device, stream) workspace, grown on demand (plumbing, not compute).

    Zero-filled when allocated: its first 8 KiB hold the library's split-K
    counters, which must start at zero and which every call leaves at zero.
    A workspace that is outgrown is kept alive, never returned to torch's
    allocator: a HIP graph captured earlier on the stream still holds its
    address and writes its counters and partials there on every replay."""
    key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
    buf = _ws.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _ws_retired.append(buf)
        buf = torch.zeros(max(nbytes, 16384), dtype=torch.uint8, device=device)
        _ws[key] = buf
    return buf


def _opts(gamma, eps, perm, residue_cols, static_scale, smooth=None):
    if gamma is None and perm is None and not residue_cols and static_scale is None and smooth is None:
        return None, []
    keep = []
    if smooth is not None:
        assert smooth.dtype == torch.float32 and smooth.is_contiguous()
        keep.append(smooth)
    if gamma is not None:
        assert gamma.dtype == torch.bfloat16 and gamma.is_contiguous()
        keep.append(gamma)
    if perm is not None:
        assert perm.dtype == torch.int32 and perm.is_contiguous()
        keep.append(perm)
    if static_scale is not None:
        if not torch.is_tensor(static_scale):
            static_scale = torch.tensor([float(static_scale)], dtype=torch.float32,
                                        device=(gamma if gamma is not None else perm).device
                                        if (gamma is not None or perm is not None) else "cuda")
        keep.append(static_scale)
    o = _COpts(_ptr(gamma), C.c_float(eps), _ptr(perm), int(residue_cols), _ptr(static_scale), _ptr(smooth))
    return o, keep


def quantize(x: torch.Tensor, gamma=None, eps: float = 1e-6, perm=None, residue_cols: int = 0,
             static_scale=None, smooth=None) -> NVFP4Tensor:
    """NVFP4-quantize rows of x (bf16/f32, 2-D), optionally fused with RMSNorm, a diagonal
    smoothing multiply, a channel gather and residue columns; returns rows x (K + residue_cols)."""
    assert x.dim() == 2 and x.stride(1) == 1
    rows, K = x.shape
    out = NVFP4Tensor.empty(rows, K + residue_cols, x.device)
    o, keep = _opts(gamma, eps, perm, residue_cols, static_scale, smooth)
    n = lib().nvfp4_workspace_size(0, rows, 0, K, residue_cols)
    ws = workspace(n, x.device)
    ct = out.c()
    _check(lib().nvfp4_quantize(_ptr(x), _dtype_code(x), rows, K, x.stride(0),
                                C.byref(o) if o is not None else None, C.byref(ct),
                                _ptr(ws), ws.numel(), _stream()), "nvfp4_quantize")
    return out


def gemm(a, w: NVFP4Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """y = Q(a) Q(w)^T; a is an NVFP4Tensor or a raw bf16/f32 [M, K] tensor (quantized in the call)."""
    N, K = w.rows, w.K
    if isinstance(a, NVFP4Tensor):
        M, dev = a.rows, a.codes.device
    else:
        assert a.dim() == 2 and a.stride(1) == 1
        M, dev = a.shape[0], a.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    yt = _dtype_code(out)
    if isinstance(a, NVFP4Tensor):
        ac = a.c()
        n = lib().nvfp4_workspace_size(1, M, N, K, 0)
        ws = workspace(n, dev)
        _check(lib().nvfp4_gemm(C.byref(ac), None, 0, M, K, 0, C.byref(w.c()), _ptr(out), yt, out.stride(0),
                                _ptr(ws), ws.numel(), _stream()), "nvfp4_gemm")
    else:
        n = lib().nvfp4_workspace_size(1, M, N, K, 0)
        ws = workspace(n, dev)
        _check(lib().nvfp4_gemm(None, _ptr(a), _dtype_code(a), M, K, a.stride(0), C.byref(w.c()), _ptr(out),
                                yt, out.stride(0), _ptr(ws), ws.numel(), _stream()), "nvfp4_gemm")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def gemm_noalloc(a, w: NVFP4Tensor, out: torch.Tensor) -> torch.Tensor:
    """nvfp4_gemm_noalloc: y = Q(a) Q(w)^T into the caller's `out` with no workspace
    (the library's static per-GPU scratch); a is an NVFP4Tensor or a raw bf16/f32 tensor."""
    N, K = w.rows, w.K
    yt = _dtype_code(out)
    if isinstance(a, NVFP4Tensor):
        ac = a.c()
        _check(lib().nvfp4_gemm_noalloc(C.byref(ac), None, 0, a.rows, K, 0, C.byref(w.c()), _ptr(out), yt,
                                        out.stride(0), _stream()), "nvfp4_gemm_noalloc")
    else:
        assert a.dim() == 2 and a.stride(1) == 1
        _check(lib().nvfp4_gemm_noalloc(None, _ptr(a), _dtype_code(a), a.shape[0], K, a.stride(0), C.byref(w.c()),
                                        _ptr(out), yt, out.stride(0), _stream()), "nvfp4_gemm_noalloc")
    return out


def gemm_residue(x: torch.Tensor, w: NVFP4Tensor, residue_cols: int, gamma=None, eps: float = 1e-6,
                 perm=None, static_scale=None, out_dtype=torch.float32, return_aug: bool = False,
                 out: torch.Tensor | None = None, smooth=None):
    """Y = s_aug [Q(X') | Q(R)] [Q(W) | Q(W[:, :S])]^T with X' = perm/RMSNorm(x), R its residue
    on columns [0, S). w must already be in the channel order of perm."""
    assert x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    N = w.rows
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    o, keep = _opts(gamma, eps, perm, residue_cols, static_scale, smooth)
    if o is None:
        o = _COpts(None, C.c_float(eps), None, 0, None, None)
    aug = NVFP4Tensor.empty(M, K + residue_cols, x.device) if return_aug else None
    augc = aug.c() if aug is not None else None
    n = lib().nvfp4_workspace_size(2, M, N, K, residue_cols)
    ws = workspace(n, x.device)
    _check(lib().nvfp4_gemm_residue(_ptr(x), _dtype_code(x), M, K, x.stride(0), C.byref(o), C.byref(w.c()),
                                    _ptr(out), _dtype_code(out), out.stride(0),
                                    C.byref(augc) if augc is not None else None,
                                    _ptr(ws), ws.numel(), _stream()), "nvfp4_gemm_residue")
    return (out, aug) if return_aug else out


def channel_absmax(x: torch.Tensor, gamma=None, eps: float = 1e-6) -> torch.Tensor:
    assert x.dim() == 2 and x.stride(1) == 1
    rows, K = x.shape
    out = torch.empty((K,), dtype=torch.float32, device=x.device)
    n = lib().nvfp4_workspace_size(3, rows, 0, K, 0)
    ws = workspace(n, x.device)
    _check(lib().nvfp4_channel_absmax(_ptr(x), _dtype_code(x), rows, K, x.stride(0), _ptr(gamma),
                                      C.c_float(eps), _ptr(out), _ptr(ws), ws.numel(), _stream()),
           "nvfp4_channel_absmax")
    return out


def perm_from_absmax(v: torch.Tensor) -> torch.Tensor:
    """Host sort: channels by descending absmax, ties by ascending index (int32, on v's device)."""
    vh = v.detach().float().cpu().contiguous()
    p = torch.empty(vh.numel(), dtype=torch.int32)
    _check(lib().nvfp4_perm_from_absmax(C.c_void_p(vh.data_ptr()), vh.numel(), C.c_void_p(p.data_ptr())),
           "nvfp4_perm_from_absmax")
    return p.to(v.device)


def calibrate_perm(x_cal: torch.Tensor, gamma=None, eps: float = 1e-6) -> torch.Tensor:
    return perm_from_absmax(channel_absmax(x_cal, gamma, eps))


# ---------------------------------------------------------------------- MXFP4

class _CMXTensor(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("ld_codes", C.c_int64), ("scales", C.c_void_p),
                ("ld_scales", C.c_int64), ("rows", C.c_int64), ("K", C.c_int64), ("layout", C.c_int32)]


class MXTensor:
    """Device MXFP4 tensor: codes [rows, ld_codes] u8 (E2M1 nibbles), scales [rows, ld_scales]
    u8 (E8M0, one per 32 columns); no tensor scale. A tiled tensor (layout 1, weights of the
    M <= 64 product) stores ceil(rows/16) strips of ld_codes / ld_scales bytes and keeps its
    logical row count in `nrows`."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, K: int, layout: int = ROWMAJOR,
                 nrows: int | None = None):
        self.codes, self.scales, self.K, self.layout = codes, scales, K, layout
        self.nrows = codes.shape[0] if nrows is None else nrows

    @staticmethod
    def empty(rows: int, K: int, device="cuda") -> "MXTensor":
        ldc, lds = _round_up(max(K // 2, 1), 16), _round_up(max(K // 32, 1), 16)
        return MXTensor(torch.empty((rows, ldc), dtype=torch.uint8, device=device),
                        torch.empty((rows, lds), dtype=torch.uint8, device=device), K)

    @staticmethod
    def empty_tiled(rows: int, K: int, device="cuda") -> "MXTensor":
        ku, nt = max((K + 511) // 512, 1), max((rows + 15) // 16, 1)
        return MXTensor(torch.empty((nt, ku * 4096), dtype=torch.uint8, device=device),
                        torch.empty((nt, ku * 256), dtype=torch.uint8, device=device), K, TILED, rows)

    @property
    def rows(self) -> int:
        return self.nrows

    def c(self) -> _CMXTensor:
        return _CMXTensor(self.codes.data_ptr(), self.codes.stride(0), self.scales.data_ptr(), self.scales.stride(0),
                          self.rows, self.K, self.layout)

    def host(self):
        """(codes [rows, K/2], scales [rows, K/32]) as numpy arrays on the host (row-major only)."""
        assert self.layout == ROWMAJOR, "host() reads the row-major layout"
        return self.codes[:, : self.K // 2].cpu().numpy(), self.scales[:, : self.K // 32].cpu().numpy()


def mx_quantize(x: torch.Tensor, residue_cols: int = 0) -> MXTensor:
    """MXFP4-quantize rows of x (bf16/f32, 2-D, K % 32 == 0); residue_cols > 0 appends the
    quantized residue of the first residue_cols columns."""
    assert x.dim() == 2 and (x.stride(1) == 1 or x.numel() == 0)
    rows, K = x.shape
    out = MXTensor.empty(rows, K + residue_cols, x.device)
    ct = out.c()
    _check(lib().nvfp4_mx_quantize(_ptr(x), _dtype_code(x), rows, K, max(x.stride(0), K), int(residue_cols), C.byref(ct),
                                   _stream()), "nvfp4_mx_quantize")
    return out


def mx_pack_tiled(w: MXTensor) -> MXTensor:
    """The tiled copy of a row-major MXFP4 weight (nvfp4_mx_pack_tiled), on the current stream."""
    out = MXTensor.empty_tiled(w.rows, w.K, device=w.codes.device)
    src, dst = w.c(), out.c()
    _check(lib().nvfp4_mx_pack_tiled(C.byref(src), C.byref(dst), _stream()), "nvfp4_mx_pack_tiled")
    return out


def mx_gemm(a: MXTensor, w: MXTensor, residue_cols: int = 0, out_dtype=torch.float32,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """y = A W^T in MXFP4; A has K + residue_cols columns, W has K."""
    M, N = a.rows, w.rows
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.codes.device)
    n = lib().nvfp4_workspace_size(4, M, N, w.K, residue_cols)
    ws = workspace(n, a.codes.device) if n else None
    ac, wc = a.c(), w.c()
    _check(lib().nvfp4_mx_gemm(C.byref(ac), C.byref(wc), int(residue_cols), _ptr(out), _dtype_code(out),
                               out.stride(0), _ptr(ws), ws.numel() if ws is not None else 0, _stream()),
           "nvfp4_mx_gemm")
    return out


def decode_attention(q: torch.Tensor, k_cache: NVFP4Tensor, vt_cache: NVFP4Tensor, T: int,
                     compensate: bool = True, out: torch.Tensor | None = None) -> torch.Tensor:
    """nvfp4_decode_attention: q [H, D] (bf16/f32); k_cache NVFP4 [H*T, D]; vt_cache NVFP4
    [H*D, T] (V transposed); returns o [H, D] FP32. compensate adds the residue columns of
    the query and of the probabilities."""
    assert q.dim() == 2 and q.stride(1) == 1
    H, D = q.shape
    if out is None:
        out = torch.empty((H, D), dtype=torch.float32, device=q.device)
    n = lib().nvfp4_workspace_size(5, H, D, T, 0)
    ws = workspace(n, q.device)
    kc, vc = k_cache.c(), vt_cache.c()
    _check(lib().nvfp4_decode_attention(_ptr(q), _dtype_code(q), H, D, q.stride(0), C.byref(kc), C.byref(vc),
                                        int(T), 1 if compensate else 0, _ptr(out), out.stride(0), _ptr(ws),
                                        ws.numel(), _stream()), "nvfp4_decode_attention")
    return out
