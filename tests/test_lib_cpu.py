"""Host-side checks of libnvfp4 that need no GPU: the library loads, exports every
entry point declared in include/nvfp4.h, its argument checks reject bad calls
before touching the device, and the kernels' scalar rounding helpers (built for
the host from the same source) agree bit for bit with the oracle."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from block_scaled_fp4_02_amd import build, nvfp4
    build.build(force=False)
    return nvfp4.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    from block_scaled_fp4_02_amd import nvfp4
    assert sorted(nvfp4.EXPORTS) == names


def test_version_and_strings(L):
    assert L.nvfp4_version() == 10300
    assert L.nvfp4_status_string(0) == b"ok"
    assert L.nvfp4_status_string(5) == b"workspace too small"


def test_host_e4m3_matches_oracle(L, orc):
    rng = np.random.default_rng(5)
    finite = np.array([orc.e4m3_value(b) for b in range(127)])
    mids = (finite[:-1] + finite[1:]) / 2
    vals = np.concatenate([finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                           2.0 ** rng.uniform(-30, 12, 20000), rng.uniform(0, 500, 5000),
                           [0.0, 1e-45, 2.0 ** -10, 448.0, 463.99, 464.0, 1e30]]).astype(np.float32)
    for v in vals:
        assert L.nvfp4_host_e4m3_encode(C.c_float(v)) == orc.e4m3_encode(v), v


def test_host_e2m1_matches_oracle(L, orc):
    rng = np.random.default_rng(6)
    book = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = (book[:-1] + book[1:]) / 2
    q = np.concatenate([book, mids, np.nextafter(mids, 0), np.nextafter(mids, 9), rng.uniform(-8, 8, 20000),
                        [0.0, -0.0, 6.4, 1e30, -1e30, 1e-40]]).astype(np.float32)
    q = np.concatenate([q, -q])
    for v in q:
        assert L.nvfp4_host_e2m1_encode(C.c_float(v)) == orc.e2m1_encode(v), v


def test_workspace_sizes(L):
    assert L.nvfp4_workspace_size(0, 4, 0, 64, 0) > 0
    assert L.nvfp4_workspace_size(1, 16, 14336, 4096, 0) >= 16 * 2048
    assert L.nvfp4_workspace_size(2, 16, 8192, 8192, 8192) > L.nvfp4_workspace_size(1, 16, 8192, 8192, 0)
    assert L.nvfp4_workspace_size(9, 1, 1, 16, 0) == 0


def _tensor(rows, K, codes=16, scales=16, scale=16, ldc=None, lds=None, layout=0):
    from block_scaled_fp4_02_amd.nvfp4 import _CTensor
    if layout == 1:
        ku = (K + 511) // 512
        dl, ds = ku * 4096, ku * 512
    else:
        dl, ds = max(16, (K // 2 + 15) // 16 * 16), max(8, (K // 16 + 7) // 8 * 8)
    return _CTensor(codes, ldc if ldc is not None else dl, scales, lds if lds is not None else ds, scale, rows, K,
                    layout)


def test_argument_errors_before_launch(L):
    """Bad arguments come back as status codes; fake (never dereferenced) pointers."""
    vp = C.c_void_p
    fake = vp(1 << 20)
    out = _tensor(4, 64, codes=1 << 20, scales=1 << 21, scale=1 << 22)
    ws, wsn = fake, 1 << 20
    # null input
    assert L.nvfp4_quantize(None, 0, 4, 64, 64, None, C.byref(out), ws, wsn, None) == 1
    # K not a multiple of 16
    assert L.nvfp4_quantize(fake, 0, 4, 60, 64, None, C.byref(out), ws, wsn, None) == 2
    # bad dtype
    assert L.nvfp4_quantize(fake, 7, 4, 64, 64, None, C.byref(out), ws, wsn, None) == 4
    # misaligned input
    assert L.nvfp4_quantize(vp((1 << 20) + 2), 0, 4, 64, 64, None, C.byref(out), ws, wsn, None) == 3
    # output shape mismatch
    bad = _tensor(5, 64, codes=1 << 20, scales=1 << 21, scale=1 << 22)
    assert L.nvfp4_quantize(fake, 0, 4, 64, 64, None, C.byref(bad), ws, wsn, None) == 2
    # misaligned leading dimension of codes
    bad = _tensor(4, 64, codes=1 << 20, scales=1 << 21, scale=1 << 22, ldc=40)
    assert L.nvfp4_quantize(fake, 0, 4, 64, 64, None, C.byref(bad), ws, wsn, None) == 3
    # workspace too small
    assert L.nvfp4_quantize(fake, 0, 4, 64, 64, None, C.byref(out), ws, 16, None) == 5
    # gemm: both or neither activation source
    w = _tensor(32, 64, codes=1 << 20, scales=1 << 21, scale=1 << 22)
    assert L.nvfp4_gemm(None, None, 0, 4, 64, 64, C.byref(w), fake, 1, 32, ws, wsn, None) == 1
    assert L.nvfp4_gemm(C.byref(out), fake, 0, 4, 64, 64, C.byref(w), fake, 1, 32, ws, wsn, None) == 1
    # gemm: K mismatch between activation and weight
    w2 = _tensor(32, 48, codes=1 << 20, scales=1 << 21, scale=1 << 22)
    assert L.nvfp4_gemm(C.byref(out), None, 0, 4, 64, 0, C.byref(w2), fake, 1, 32, ws, wsn, None) == 2
    # gemm: ldy too small, bad output dtype
    assert L.nvfp4_gemm(C.byref(out), None, 0, 4, 64, 0, C.byref(w), fake, 1, 16, ws, wsn, None) == 2
    assert L.nvfp4_gemm(C.byref(out), None, 0, 4, 64, 0, C.byref(w), fake, 3, 32, ws, wsn, None) == 4
    # residue: S not a multiple of 16 / larger than K
    from block_scaled_fp4_02_amd.nvfp4 import _COpts
    o = _COpts(None, C.c_float(1e-6), None, 24, None)
    assert L.nvfp4_gemm_residue(fake, 0, 4, 64, 64, C.byref(o), C.byref(w), fake, 1, 32, None, ws, wsn, None) == 2
    o = _COpts(None, C.c_float(1e-6), None, 80, None)
    assert L.nvfp4_gemm_residue(fake, 0, 4, 64, 64, C.byref(o), C.byref(w), fake, 1, 32, None, ws, wsn, None) == 2
    # permutation pointer not 16-byte aligned (the quantizer reads it as 16-byte vectors)
    o = _COpts(None, C.c_float(1e-6), vp((1 << 20) + 4), 0, None)
    assert L.nvfp4_quantize(fake, 0, 4, 64, 64, C.byref(o), C.byref(out), ws, wsn, None) == 3
    assert L.nvfp4_gemm_residue(fake, 0, 4, 64, 64, C.byref(o), C.byref(w), fake, 1, 32, None, ws, wsn, None) == 3
    # smoothing vector not 16-byte aligned
    o = _COpts(None, C.c_float(1e-6), None, 0, None, vp((1 << 20) + 8))
    assert L.nvfp4_quantize(fake, 0, 4, 64, 64, C.byref(o), C.byref(out), ws, wsn, None) == 3
    # permutation beyond the staged-row limit
    o = _COpts(None, C.c_float(1e-6), fake, 0, None)
    assert L.nvfp4_quantize(fake, 0, 4, 32784, 32784, C.byref(o),
                            C.byref(_tensor(4, 32784, codes=1 << 20, scales=1 << 21, scale=1 << 22)),
                            ws, 1 << 30, None) == 6


def test_tiled_layout_argument_errors(L):
    """The tiled layout is accepted for weights only, with its fixed strides."""
    vp = C.c_void_p
    fake = vp(1 << 20)
    ws, wsn = fake, 1 << 20
    a = _tensor(4, 1024, codes=1 << 20, scales=1 << 21, scale=1 << 22)
    wt = _tensor(32, 1024, codes=1 << 23, scales=1 << 24, scale=1 << 25, layout=1)
    # tiled activations are not supported
    at = _tensor(4, 1024, codes=1 << 20, scales=1 << 21, scale=1 << 22, layout=1)
    assert L.nvfp4_gemm(C.byref(at), None, 0, 4, 1024, 0, C.byref(wt), fake, 1, 32, ws, wsn, None) == 6
    # wrong strip strides / unknown layout code
    bad = _tensor(32, 1024, codes=1 << 23, scales=1 << 24, scale=1 << 25, layout=1, ldc=4096)
    assert L.nvfp4_gemm(C.byref(a), None, 0, 4, 1024, 0, C.byref(bad), fake, 1, 32, ws, wsn, None) == 2
    bad = _tensor(32, 1024, codes=1 << 23, scales=1 << 24, scale=1 << 25, layout=1, lds=8192)
    assert L.nvfp4_gemm(C.byref(a), None, 0, 4, 1024, 0, C.byref(bad), fake, 1, 32, ws, wsn, None) == 2
    bad = _tensor(32, 1024, codes=1 << 23, scales=1 << 24, scale=1 << 25, layout=5)
    assert L.nvfp4_gemm(C.byref(a), None, 0, 4, 1024, 0, C.byref(bad), fake, 1, 32, ws, wsn, None) == 2
    # misaligned tiled codes
    bad = _tensor(32, 1024, codes=(1 << 23) + 8, scales=1 << 24, scale=1 << 25, layout=1)
    assert L.nvfp4_gemm(C.byref(a), None, 0, 4, 1024, 0, C.byref(bad), fake, 1, 32, ws, wsn, None) == 3
    # pack: source must be row-major, destination tiled with the same shape
    w = _tensor(32, 1024, codes=1 << 20, scales=1 << 21, scale=1 << 22)
    assert L.nvfp4_pack_tiled(C.byref(wt), C.byref(wt), None) == 6
    assert L.nvfp4_pack_tiled(C.byref(w), C.byref(a), None) == 2
    assert L.nvfp4_pack_tiled(C.byref(w), C.byref(_tensor(48, 1024, codes=1 << 23, scales=1 << 24,
                                                           scale=1 << 25, layout=1)), None) == 2
    assert L.nvfp4_pack_tiled(None, C.byref(wt), None) == 1


def test_perm_from_absmax_host(L, orc):
    rng = np.random.default_rng(9)
    v = rng.integers(0, 30, 500).astype(np.float32)
    p = np.zeros(500, np.int32)
    assert L.nvfp4_perm_from_absmax(C.c_void_p(v.ctypes.data), 500, C.c_void_p(p.ctypes.data)) == 0
    assert np.array_equal(p, orc.perm_from_absmax(v))


def test_noalloc_rejects_oversized_before_launch(L):
    """nvfp4_gemm_noalloc refuses a product whose workspace exceeds the static scratch,
    before touching the device, and says how much it needs (fake pointers)."""
    vp = C.c_void_p
    fake = vp(1 << 20)
    M, N, K = 512, 8192, 28672
    assert L.nvfp4_workspace_size(1, M, N, K, 0) > (32 << 20)
    w = _tensor(N, K, codes=1 << 20, scales=1 << 21, scale=1 << 22)
    assert L.nvfp4_gemm_noalloc(None, fake, 0, M, K, K, C.byref(w), fake, 1, N, None) == 5
    assert b"static scratch" in L.nvfp4_last_error()
    # argument errors come first, as in nvfp4_gemm
    assert L.nvfp4_gemm_noalloc(None, None, 0, M, K, K, C.byref(w), fake, 1, N, None) == 1


def test_decode_attention_argument_errors(L):
    """nvfp4_decode_attention rejects bad sizes, dtypes, caches and workspaces before
    anything is enqueued (fake, never dereferenced pointers)."""
    vp = C.c_void_p
    fake = vp(1 << 20)
    H, D, T = 2, 64, 32
    kc = _tensor(H * T, D, codes=1 << 20, scales=1 << 21, scale=1 << 22)
    vt = _tensor(H * D, T, codes=1 << 23, scales=1 << 24, scale=1 << 25)
    n = L.nvfp4_workspace_size(5, H, D, T, 0)
    assert n > 8192
    ws = fake

    def call(q=fake, qt=0, h=H, d=D, ldq=D, k=kc, v=vt, t=T, comp=1, out=fake, ldo=D, wsn=n):
        return L.nvfp4_decode_attention(q, qt, h, d, ldq, C.byref(k), C.byref(v), t, comp, out, ldo, ws, wsn, None)

    assert call(qt=5) == 4                                        # dtype
    assert call(d=48) == 2 and call(d=16) == 2 and call(d=288) == 2   # D % 32, 32 <= D <= 256
    assert call(t=0) == 2 and call(t=24) == 2                     # T > 0, T % 16
    assert call(comp=2) == 2
    assert call(k=_tensor(H * T + 1, D, codes=1 << 20, scales=1 << 21, scale=1 << 22)) == 2
    assert call(v=_tensor(H * D, T + 16, codes=1 << 23, scales=1 << 24, scale=1 << 25)) == 2
    assert call(q=None) == 1 and call(out=None) == 1
    assert call(ldq=32) == 2 and call(ldo=32) == 2
    assert call(q=vp((1 << 20) + 2)) == 3
    assert call(wsn=n - 1) == 5
    assert call(h=0, k=_tensor(0, D, codes=1 << 20, scales=1 << 21, scale=1 << 22),
                v=_tensor(0, T, codes=1 << 23, scales=1 << 24, scale=1 << 25)) == 0   # nothing to do


def _mx(rows, K, codes=1 << 20, scales=1 << 21, ldc=None, lds=None, layout=0):
    from block_scaled_fp4_02_amd.nvfp4 import _CMXTensor
    if layout == 1:
        ku = (K + 511) // 512
        dl, ds = ku * 4096, ku * 256
    else:
        dl, ds = max(16, (K // 2 + 15) // 16 * 16), max(1, K // 32)
    return _CMXTensor(codes, ldc if ldc is not None else dl, scales, lds if lds is not None else ds, rows, K, layout)


def test_mx_tiled_argument_errors(L):
    """nvfp4_mx_pack_tiled and the tiled MX weight of nvfp4_mx_gemm: layouts, strides, rows,
    alignment and the M <= 64 limit are checked before anything is enqueued (fake pointers)."""
    vp = C.c_void_p
    src = _mx(40, 1024)
    dst = _mx(40, 1024, codes=1 << 22, scales=1 << 23, layout=1)
    pack = lambda s, d: L.nvfp4_mx_pack_tiled(C.byref(s), C.byref(d), None)
    assert pack(src, _mx(40, 1024, codes=1 << 22, scales=1 << 23)) == 2               # dst not tiled
    assert pack(src, _mx(40, 1024, codes=1 << 22, scales=1 << 23, layout=1, ldc=4096)) == 2   # KU = 2: 8192
    assert pack(src, _mx(40, 1024, codes=1 << 22, scales=1 << 23, layout=1, lds=256)) == 2
    assert pack(src, _mx(41, 1024, codes=1 << 22, scales=1 << 23, layout=1)) == 2      # rows differ
    assert pack(src, _mx(40, 1024, codes=(1 << 22) + 8, scales=1 << 23, layout=1)) == 3
    assert pack(_mx(40, 1024, layout=1), dst) == 6                                   # src must be row-major
    assert pack(src, _mx(40, 1024, codes=1 << 20, scales=1 << 23, layout=1)) == 2      # in place
    assert pack(src, _mx(40, 1024, codes=1 << 22, scales=1 << 23, layout=2)) == 2      # no such layout
    y = vp(1 << 26)
    gemm = lambda a, w: L.nvfp4_mx_gemm(C.byref(a), C.byref(w), 0, y, 1, 40, None, 0, None)
    assert gemm(_mx(65, 1024, codes=1 << 24, scales=1 << 25), dst) == 6               # tiled W at M > 64
    assert gemm(_mx(8, 1024, codes=1 << 24, scales=1 << 25, layout=1), dst) == 6      # tiled A
    assert gemm(_mx(8, 1024, codes=1 << 24, scales=1 << 25), _mx(40, 1024, codes=1 << 22, scales=1 << 23,
                                                                   layout=1, ldc=4096)) == 2
