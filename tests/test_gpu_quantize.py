"""GPU parity of the quantizer (nvfp4_quantize) against the CPU oracle: codes,
block scales and the tensor scale must match bit for bit."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_02_amd import inputs
from helpers import assert_qtensor_equal, note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def nv():
    from block_scaled_fp4_02_amd import nvfp4
    nvfp4.lib()
    return nvfp4


def test_gemv_operands(nv, orc):
    x, w = inputs.gemv_4096()
    note("quantize gemv x[1x4096], W[4096x4096]")
    qx, qw = nv.quantize(x.to(DEV)), nv.quantize(w.to(DEV))
    torch.cuda.synchronize()
    assert_qtensor_equal(qx, orc.quantize(x), "x")
    assert_qtensor_equal(qw, orc.quantize(w), "W")


@pytest.mark.parametrize("rows,K", [(1, 16), (3, 48), (5, 80), (7, 1040), (33, 4112), (2, 64), (130, 272)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_shapes(nv, orc, rows, K, dtype):
    x = inputs.small_random(rows * 1000 + K, rows, K).to(dtype)
    if dtype == torch.float32:
        x = x + torch.from_numpy(np.random.default_rng(K).standard_normal((rows, K)).astype(np.float32)) * 1e-3
    note(f"quantize ragged rows={rows} K={K} {dtype}")
    q = nv.quantize(x.to(DEV))
    torch.cuda.synchronize()
    assert_qtensor_equal(q, orc.quantize(x.numpy() if dtype == torch.float32 else x), f"{rows}x{K}")


def test_block_magnitudes_and_specials(nv, orc):
    """Blocks spanning 2^-40..2^40 (zero and subnormal E4M3 scales), zeros, -0, ties."""
    rng = np.random.default_rng(77)
    rows, K = 64, 1024
    x = rng.standard_normal((rows, K)).astype(np.float32)
    mag = 2.0 ** rng.uniform(-40, 40, size=(rows, K // 16))
    x *= np.repeat(mag, 16, axis=1).astype(np.float32)
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    x[2, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, np.float32) * np.float32(2 ** -3)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    for t in (xb, torch.from_numpy(x)):
        note(f"quantize magnitudes {t.dtype}")
        q = nv.quantize(t.to(DEV))
        torch.cuda.synchronize()
        ref = orc.quantize(t.float().numpy())
        assert_qtensor_equal(q, ref, f"magnitudes {t.dtype}")
        assert (ref.scales < 8).any(), "subnormal block scales must be exercised"


def test_all_bf16_values(nv, orc):
    """Every finite bf16 bit pattern, in blocks whose maxima vary."""
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    vals = (bits[finite] << 16).view(np.float32)
    n = vals.size - vals.size % 16
    rng = np.random.default_rng(3)
    x = rng.permutation(vals[:n]).reshape(-1, 16)
    # within-tensor scale spread comes from the values themselves; also a narrow variant
    for name, t in [("all", x), ("clipped", np.clip(x, -1e4, 1e4))]:
        xt = torch.from_numpy(np.ascontiguousarray(t.reshape(-1, 256) if t.size % 256 == 0 else t))
        xt = xt.to(torch.bfloat16)
        note(f"quantize all-bf16 {name} shape={tuple(xt.shape)}")
        q = nv.quantize(xt.to(DEV))
        torch.cuda.synchronize()
        assert_qtensor_equal(q, orc.quantize(xt), name)


def test_static_scale(nv, orc):
    x = inputs.small_random(9, 8, 512)
    S_dyn = float(orc.tensor_scale(x))
    for S in (S_dyn, S_dyn / 50.0, S_dyn * 3.0):
        note(f"quantize static S={S}")
        q = nv.quantize(x.to(DEV), static_scale=torch.tensor([S], dtype=torch.float32, device=DEV))
        torch.cuda.synchronize()
        assert_qtensor_equal(q, orc.quantize(x, static_S=S), f"static {S}")


def test_zero_and_empty(nv, orc):
    x = torch.zeros((3, 64), dtype=torch.bfloat16)
    note("quantize zeros")
    q = nv.quantize(x.to(DEV))
    torch.cuda.synchronize()
    assert_qtensor_equal(q, orc.quantize(x), "zeros")
    q = nv.quantize(torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert float(q.scale.cpu()[0]) == 1.0


def test_fused_rmsnorm_perm_residue(nv, orc):
    """Config of the augmented-channel product: RMSNorm + calibration reorder + residue of top S."""
    x, g, xcal, _ = inputs.outlier_aug(rows=64, N=16, cal_rows=512)
    note("calibration absmax on GPU")
    v_gpu = nv.channel_absmax(xcal.to(DEV), g.to(DEV), 1e-6)
    torch.cuda.synchronize()
    v_ref = orc.channel_absmax(xcal, g, 1e-6)
    assert np.array_equal(v_gpu.cpu().numpy(), v_ref)
    perm = orc.perm_from_absmax(v_ref)
    assert np.array_equal(nv.perm_from_absmax(v_gpu).cpu().numpy(), perm)
    pd = torch.from_numpy(perm).to(DEV)
    for S in (0, 128, 256, 512):
        note(f"quantize fused rmsnorm+perm+residue S={S}")
        q = nv.quantize(x.to(DEV), gamma=g.to(DEV), eps=1e-6, perm=pd, residue_cols=S)
        torch.cuda.synchronize()
        ref = orc.quantize_aug(x, gamma=g, eps=1e-6, perm=perm, S_cols=S)
        assert_qtensor_equal(q, ref, f"fused S={S}")
    # each step alone: norm only, perm only
    note("quantize rmsnorm only / perm only")
    q = nv.quantize(x.to(DEV), gamma=g.to(DEV), eps=1e-6)
    torch.cuda.synchronize()
    assert_qtensor_equal(q, orc.quantize_aug(x, gamma=g, eps=1e-6), "norm only")
    q = nv.quantize(x.to(DEV), perm=pd, residue_cols=64)
    torch.cuda.synchronize()
    assert_qtensor_equal(q, orc.quantize_aug(x, perm=perm, S_cols=64), "perm only")


def test_residue_k_to_2k(nv, orc):
    x, _ = inputs.residue_8192(16)
    note("quantize residue K->2K 16x8192")
    q = nv.quantize(x.to(DEV), residue_cols=8192)
    torch.cuda.synchronize()
    assert_qtensor_equal(q, orc.quantize_aug(x, S_cols=8192), "K->2K")


@pytest.mark.parametrize("shape_idx,M", [(0, 2048), (1, 8192)])
def test_prefill_activation_sampled(nv, orc, shape_idx, M):
    """Full-size prefill activations; the oracle checks sampled rows with the tensor scale it
    computes over the whole tensor."""
    K, _ = inputs.PREFILL_SHAPES[shape_idx]
    x = inputs.activations(5, shape_idx, M, K, 0.01, 50.0)
    note(f"quantize prefill activations {M}x{K}")
    q = nv.quantize(x.to(DEV))
    torch.cuda.synchronize()
    S = orc.tensor_scale(x)
    codes, scales, Sg = q.host()
    assert Sg == S
    rows = np.random.default_rng(shape_idx).choice(M, 24, replace=False)
    ref = orc.quantize(x[rows], static_S=float(S))
    assert np.array_equal(codes[rows], ref.codes) and np.array_equal(scales[rows], ref.scales)


def test_deterministic(nv):
    x, _ = inputs.decode_sweep(0)
    a = nv.quantize(x.to(DEV), residue_cols=256)
    b = nv.quantize(x.to(DEV), residue_cols=256)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales) and torch.equal(a.scale, b.scale)


@pytest.mark.parametrize("rows,K,S,dt", [(16, 14336, 0, "bf16"), (7, 4112, 2048, "bf16"), (32, 8192, 8192, "bf16"),
                                        # 32768 and 21504 blocks on 64 workgroups: two blocks per thread
                                        # (all threads, then the first 80 of each workgroup)
                                        (32, 16384, 0, "bf16"), (24, 14336, 4096, "bf16"), (24, 14336, 4096, "f32")])
def test_small_quantizer_wait_fallback(nv, orc, rows, K, S, dt, monkeypatch):
    """The one-launch quantizer of decode-sized activations, with its grid-wide
    arrival forced to give up at once (spin limit 0, set from the host): every
    workgroup then recomputes amax(X) itself. Codes must equal the oracle's."""
    x = inputs.small_random(300 + rows, rows, K)
    if dt == "f32":
        x = x.float()
    ox = orc.quantize_aug(x, S_cols=S) if S else orc.quantize(x)
    note(f"small quantizer rows={rows} K={K} S={S}: normal")
    q0 = nv.quantize(x.to(DEV), residue_cols=S)
    torch.cuda.synchronize()
    assert_qtensor_equal(q0, ox, "normal")
    monkeypatch.setenv("NVFP4_SPIN_LIMIT", "0")
    note(f"small quantizer rows={rows} K={K} S={S}: fallback")
    q1 = nv.quantize(x.to(DEV), residue_cols=S)
    torch.cuda.synchronize()
    monkeypatch.delenv("NVFP4_SPIN_LIMIT")
    assert_qtensor_equal(q1, ox, "fallback")


@pytest.mark.parametrize("rows,K,S", [(512, 8192, 0), (130, 4112, 2048), (2048, 8192, 512), (40, 28672, 0)])
def test_grid_quantizer(nv, orc, rows, K, S, monkeypatch):
    """The one-launch quantizer of mid-size activations (up to 16 M elements, X held in
    registers over a grid-wide arrival for amax(X)), at prefill and ragged shapes, with and
    without residue columns, then with the arrival forced to give up at once (spin limit 0,
    set from the host): every workgroup recomputes amax(X) itself. Codes must equal the
    oracle's both times, and a second call (the slots' next epoch) again."""
    x = inputs.small_random(700 + rows, rows, K)
    ox = orc.quantize_aug(x, S_cols=S) if S else orc.quantize(x)
    xd = x.to(DEV)
    for i in range(2):
        note(f"grid quantizer rows={rows} K={K} S={S}: call {i}")
        q0 = nv.quantize(xd, residue_cols=S)
        torch.cuda.synchronize()
        assert_qtensor_equal(q0, ox, f"call {i}")
    monkeypatch.setenv("NVFP4_SPIN_LIMIT", "0")
    note(f"grid quantizer rows={rows} K={K} S={S}: fallback")
    q1 = nv.quantize(xd, residue_cols=S)
    torch.cuda.synchronize()
    monkeypatch.delenv("NVFP4_SPIN_LIMIT")
    assert_qtensor_equal(q1, ox, "fallback")


@pytest.mark.parametrize("rows,norm,use_perm,S", [(64, True, True, 256), (7, True, True, 0), (1, True, False, 64),
                                                  (33, False, True, 512)])
def test_rows_quantizer_wait_fallback(nv, orc, rows, norm, use_perm, S, monkeypatch):
    """The one-launch quantizer of <= 64 rows with RMSNorm and/or reorder (one
    workgroup per row), normally and with its grid-wide arrival forced to give
    up at once (spin limit 0, set from the host): every workgroup then
    recomputes each row's maximum itself. Codes must equal the oracle's."""
    x, g, xcal, _ = inputs.outlier_aug(rows=64, N=16, cal_rows=64)
    x = x[:rows].contiguous()
    perm = orc.perm_from_absmax(orc.channel_absmax(xcal, g, 1e-6)) if use_perm else None
    kw = dict(residue_cols=S)
    if norm:
        kw.update(gamma=g.to(DEV), eps=1e-6)
    if use_perm:
        kw.update(perm=torch.from_numpy(perm).to(DEV))
    ref = orc.quantize_aug(x, gamma=g if norm else None, eps=1e-6, perm=perm, S_cols=S)
    note(f"row quantizer rows={rows} norm={norm} perm={use_perm} S={S}: normal")
    q0 = nv.quantize(x.to(DEV), **kw)
    torch.cuda.synchronize()
    assert_qtensor_equal(q0, ref, "normal")
    monkeypatch.setenv("NVFP4_SPIN_LIMIT", "0")
    note(f"row quantizer rows={rows} norm={norm} perm={use_perm} S={S}: fallback")
    q1 = nv.quantize(x.to(DEV), **kw)
    torch.cuda.synchronize()
    monkeypatch.delenv("NVFP4_SPIN_LIMIT")
    assert_qtensor_equal(q1, ref, "fallback")


@pytest.mark.parametrize("rows,norm,K", [(4, True, 16384), (70, False, 16384), (4, True, 28672), (70, True, 32768)])
def test_row_staging_at_large_k(nv, orc, rows, norm, K):
    """The reorder kernels stage a whole row (K floats) in LDS: at K = 16384 that
    is 64 KiB plus the kernel's own words, at 32768 (the limit) 128 KiB. Up to
    K = 16384, 4 rows take the one-launch row quantizer (RMSNorm + reorder +
    residue); 70 rows, and longer rows, the two-pass gather path."""
    x = inputs.small_random(400 + rows, rows, K)
    g = inputs.gamma(9, 0, K)
    perm = np.random.default_rng([0, 102, rows]).permutation(K).astype(np.int32)
    S = 512 if norm else 0
    kw = dict(perm=torch.from_numpy(perm).to(DEV), residue_cols=S)
    if norm:
        kw.update(gamma=g.to(DEV), eps=1e-6)
    note(f"row staging rows={rows} K={K} norm={norm} S={S}")
    q = nv.quantize(x.to(DEV), **kw)
    torch.cuda.synchronize()
    ref = orc.quantize_aug(x, gamma=g if norm else None, eps=1e-6, perm=perm, S_cols=S)
    assert_qtensor_equal(q, ref, f"rows={rows}")


@pytest.mark.parametrize("rows,K,norm,perm,S", [(4, 4096, False, False, 0), (64, 4096, True, True, 256),
                                                 (7, 1040, True, False, 64), (33, 2048, False, True, 0),
                                                 (130, 4096, True, True, 512), (300, 1024, False, False, 0),
                                                 (130, 528, True, False, 528), (20, 20000, False, False, 0)])
def test_smoothing_fused(nv, orc, rows, K, norm, perm, S):
    """Diagonal smoothing inside the fused quantizer (per input channel, after RMSNorm,
    before the reorder): every kernel path -- one workgroup per row (rows <= 64,
    K <= 16384), the two-pass amax + encode and the row-gather path -- bit for bit."""
    x = inputs.small_random(900 + rows + K, rows, K)
    sm = np.random.default_rng(K + rows).uniform(0.125, 8.0, K).astype(np.float32)
    g = inputs.gamma(9, rows, K) if norm else None
    p = np.random.default_rng(rows).permutation(K).astype(np.int32) if perm else None
    note(f"quantize smoothing rows={rows} K={K} norm={norm} perm={perm} S={S}")
    q = nv.quantize(x.to(DEV), gamma=g.to(DEV) if norm else None, eps=1e-6,
                    perm=torch.from_numpy(p).to(DEV) if perm else None, residue_cols=S,
                    smooth=torch.from_numpy(sm).to(DEV))
    torch.cuda.synchronize()
    ref = orc.quantize_aug(x, gamma=g, eps=1e-6, perm=p, S_cols=S, smooth=sm)
    assert_qtensor_equal(q, ref, "smoothed")
