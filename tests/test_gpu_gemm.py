"""GPU parity of the W4A4 products (nvfp4_gemm, nvfp4_gemm_residue) against the
FP64 oracle. Bar: the floored relative error max|y - y*| / max(|y*|, 1e-3 max|y*|)
stays within 2e-3 (FP32 accumulation of exact products); BF16 outputs may add
half a bf16 ulp. The quantized operands are checked bit for bit on the way."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_02_amd import inputs
from helpers import assert_qtensor_equal, bf16_bound_ok, gemm_error, note, untile

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


@pytest.fixture(scope="module")
def nv():
    from block_scaled_fp4_02_amd import nvfp4
    nvfp4.lib()
    return nvfp4


def test_gemv_4096(nv, orc):
    x, w = inputs.gemv_4096()
    note("gemm gemv 1x4096x4096")
    wq = nv.quantize(w.to(DEV))
    y = nv.gemm(x.to(DEV), wq)
    torch.cuda.synchronize()
    ow = orc.quantize(w)
    assert_qtensor_equal(wq, ow, "W")
    ref = orc.gemm(orc.quantize(x), ow)
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, err


@pytest.mark.parametrize("shape_idx", [0, 1, 2])
def test_decode_sweep(nv, orc, shape_idx):
    K, N = inputs.DECODE_SHAPES[shape_idx]
    x, w = inputs.decode_sweep(shape_idx)
    note(f"gemm decode sweep K={K} N={N}: quantize W")
    wq = nv.quantize(w.to(DEV))
    torch.cuda.synchronize()
    ow = orc.quantize(w)
    assert_qtensor_equal(wq, ow, "W")
    xd = x.to(DEV)
    for M in inputs.DECODE_MS:
        note(f"gemm decode M={M} K={K} N={N}")
        y = nv.gemm(xd[:M], wq)
        torch.cuda.synchronize()
        ref = orc.gemm(orc.quantize(x[:M]), ow)
        err = gemm_error(y.cpu().numpy(), ref)
        assert err <= TOL, (M, err)


def test_prequantized_activation_path(nv, orc):
    x, w = inputs.decode_sweep(2)
    wq = nv.quantize(w.to(DEV))
    xq = nv.quantize(x[:8].to(DEV))
    note("gemm with pre-quantized activations")
    y1 = nv.gemm(xq, wq)
    y2 = nv.gemm(x[:8].to(DEV), wq)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("M", inputs.RESIDUE_MS)
def test_residue_k_to_2k(nv, orc, M):
    x, w = inputs.residue_8192(16)
    x = x[:M]
    note(f"gemm_residue K->2K M={M}")
    wq = nv.quantize(w.to(DEV))
    y, aug = nv.gemm_residue(x.to(DEV), wq, 8192, return_aug=True)
    y0 = nv.gemm(x.to(DEV), wq)
    torch.cuda.synchronize()
    ref, xa, wa = orc.gemm_residue(x, w, 8192)
    assert_qtensor_equal(aug, xa, "X_aug")
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, err
    # the compensated product is closer to the product with unquantized activations
    exact = x.float().numpy().astype(np.float64) @ orc.dequantize(orc.quantize(w)).T
    e_res = np.linalg.norm(y.cpu().numpy() - exact)
    e_base = np.linalg.norm(y0.cpu().numpy() - exact)
    assert e_res <= 0.25 * e_base, (e_res, e_base)


@pytest.mark.parametrize("S", inputs.AUG_S)
def test_outlier_augmented(nv, orc, S):
    """RMSNorm + calibrated reorder + residue of the top S channels, M=64, N=14336."""
    x, g, xcal, w = inputs.outlier_aug()
    perm = orc.calibrate_perm(xcal, g)
    pd = torch.from_numpy(perm).to(DEV)
    w_perm = w[:, torch.from_numpy(perm).long()]
    note(f"gemm_residue augmented S={S}")
    wq = nv.quantize(w_perm.to(DEV))
    y, aug = nv.gemm_residue(x.to(DEV), wq, S, gamma=g.to(DEV), eps=1e-6, perm=pd, return_aug=True)
    torch.cuda.synchronize()
    xa = orc.quantize_aug(x, gamma=g, eps=1e-6, perm=perm, S_cols=S)
    assert_qtensor_equal(aug, xa, "X_aug")
    wa = orc.weight_aug(w_perm, S)
    cols = np.sort(np.random.default_rng(S).choice(14336, 1024, replace=False))
    sub = orc.QTensor(np.ascontiguousarray(wa.codes[cols]), np.ascontiguousarray(wa.scales[cols]), wa.S, wa.K)
    ref = orc.gemm(xa, sub)
    err = gemm_error(y.cpu().numpy()[:, cols], ref)
    assert err <= TOL, err


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_prefill_sampled(nv, orc, shape_idx):
    K, N = inputs.PREFILL_SHAPES[shape_idx]
    xall, w = inputs.prefill(shape_idx, 8192)
    note(f"prefill K={K} N={N}: quantize W")
    wq = nv.quantize(w.to(DEV))
    torch.cuda.synchronize()
    ow_S = orc.tensor_scale(w)
    assert float(wq.scale.cpu()[0]) == ow_S
    xd = xall.to(DEV)
    wc, ws_, _ = wq.host()
    rng = np.random.default_rng(shape_idx)
    for M in inputs.PREFILL_MS:
        note(f"prefill gemm M={M} K={K} N={N}")
        yb = nv.gemm(xd[:M], wq, out_dtype=torch.bfloat16)
        y32 = nv.gemm(xd[:M], wq, out_dtype=torch.float32) if M == 512 else None
        torch.cuda.synchronize()
        ms = rng.integers(0, M, 384)
        ns = rng.integers(0, N, 384)
        S_x = orc.tensor_scale(xall[:M])
        rows = np.unique(ms)
        xq = orc.quantize(xall[rows], static_S=float(S_x))
        pos = {r: i for i, r in enumerate(rows)}
        wrows = np.unique(ns)
        wsub = orc.quantize(w[wrows], static_S=float(ow_S))
        wpos = {r: i for i, r in enumerate(wrows)}
        # weight rows must match the device codes too
        assert np.array_equal(wsub.codes, wc[wrows]) and np.array_equal(wsub.scales, ws_[wrows])
        ref = orc.gemm_pairs(xq, wsub, np.array([pos[m] for m in ms]), np.array([wpos[n] for n in ns]))
        got = yb.float().cpu().numpy()[ms, ns]
        assert bf16_bound_ok(got, ref), (M, gemm_error(got, ref))
        if y32 is not None:
            err = gemm_error(y32.cpu().numpy()[ms, ns], ref)
            assert err <= TOL, err


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 15, 48), (16, 47, 528), (17, 300, 1040), (33, 64, 528),
                                   (64, 130, 272), (65, 47, 1040), (130, 300, 528), (5, 1000, 4112),
                                   (12, 200, 512), (12, 300, 1040)])
@pytest.mark.parametrize("S_frac", [0, 1])
def test_ragged_products(nv, orc, M, N, K, S_frac):
    x = inputs.small_random(M * 7 + K, M, K)
    w = inputs.small_random(N * 11 + K + 1, N, K, scale=0.02)
    S = 0 if S_frac == 0 else (K if K <= 528 else 256)
    note(f"ragged gemm M={M} N={N} K={K} S={S}")
    wq = nv.quantize(w.to(DEV))
    if S == 0:
        y = nv.gemm(x.to(DEV), wq)
        yb = nv.gemm(x.to(DEV), wq, out_dtype=torch.bfloat16)
        ref = orc.gemm(orc.quantize(x), orc.quantize(w))
    else:
        y = nv.gemm_residue(x.to(DEV), wq, S)
        yb = nv.gemm_residue(x.to(DEV), wq, S, out_dtype=torch.bfloat16)
        ref, _, _ = orc.gemm_residue(x, w, S)
    torch.cuda.synchronize()
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, err
    assert bf16_bound_ok(yb.float().cpu().numpy(), ref)


def test_empty_and_zero_k(nv):
    wq = nv.quantize(torch.ones((8, 32), dtype=torch.bfloat16, device=DEV))
    y = nv.gemm(torch.ones((0, 32), dtype=torch.bfloat16, device=DEV), wq)
    assert y.shape == (0, 8)
    w0 = nv.quantize(torch.ones((8, 0), dtype=torch.bfloat16, device=DEV))
    note("gemm K=0")
    y = nv.gemm(torch.ones((4, 0), dtype=torch.bfloat16, device=DEV), w0)
    torch.cuda.synchronize()
    assert not y.any()


def test_deterministic(nv):
    x, w = inputs.decode_sweep(1)
    wq = nv.quantize(w.to(DEV))
    xd = x.to(DEV)
    note("determinism")
    a = nv.gemm(xd, wq)
    b = nv.gemm(xd, wq)
    c = nv.gemm_residue(xd, wq, 4096)
    d = nv.gemm_residue(xd, wq, 4096)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


def test_graph_replay_matches_eager(nv):
    """The decode call captured in a HIP graph gives the eager result on every replay,
    with unrelated eager work and synchronizations between replays."""
    x, w = inputs.decode_sweep(0)
    xd = x.to(DEV)
    wq = nv.quantize(w.to(DEV))
    y = torch.empty((16, 14336), dtype=torch.float32, device=DEV)
    yr = torch.empty((4, 14336), dtype=torch.float32, device=DEV)
    eager = nv.gemm(xd, wq).clone()
    eager_r = nv.gemm_residue(xd[:4], wq, 4096).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        nv.gemm(xd, wq, out=y)
        nv.gemm_residue(xd[:4], wq, 4096, out=yr)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            nv.gemm(xd, wq, out=y)
            nv.gemm_residue(xd[:4], wq, 4096, out=yr)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        note(f"graph replay {i}")
        y.zero_(); yr.zero_()
        g.replay()
        other = nv.gemm(xd[:2], wq)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, eager) and torch.equal(yr, eager_r), i
        assert other.shape == (2, 14336)


@pytest.mark.parametrize("N,K", [(47, 528), (300, 1040), (4096, 4096), (33, 16)])
def test_pack_tiled_layout(nv, N, K):
    """nvfp4_pack_tiled is the documented byte permutation (checked on the host)."""
    w = inputs.small_random(70 + N, N, K)
    note(f"pack tiled N={N} K={K}")
    wq = nv.quantize(w.to(DEV))
    wt = nv.pack_tiled(wq)
    torch.cuda.synchronize()
    codes, scales, S = wq.host()
    tc, ts, pad_zero = untile(wt.codes.cpu().numpy(), wt.scales.cpu().numpy(), N, K)
    assert np.array_equal(tc, codes) and np.array_equal(ts, scales) and pad_zero
    assert wt.scale.cpu().numpy()[0] == S


@pytest.mark.parametrize("M,N,K,S", [(1, 14336, 4096, 0), (16, 4096, 14336, 0), (5, 6144, 4096, 0),
                                     (32, 300, 1040, 0), (16, 8192, 8192, 8192), (8, 1000, 4112, 2048),
                                     (64, 300, 1040, 0), (130, 47, 528, 528), (3, 15, 48, 48)])
def test_tiled_weights_same_result(nv, M, N, K, S):
    """Products with tiled weights equal those with row-major weights bit for bit
    (same arithmetic, only the load order of the weight bytes changes)."""
    x = inputs.small_random(90 + M, M, K)
    w = inputs.small_random(91 + N, N, K)
    xd = x.to(DEV)
    wq = nv.quantize(w.to(DEV))
    wt = nv.pack_tiled(wq)
    note(f"tiled weights M={M} N={N} K={K} S={S}")
    if S == 0:
        y0, y1 = nv.gemm(xd, wq), nv.gemm(xd, wt)
        aq = nv.quantize(xd)
        z0, z1 = nv.gemm(aq, wq, out_dtype=torch.bfloat16), nv.gemm(aq, wt, out_dtype=torch.bfloat16)
    else:
        y0, y1 = nv.gemm_residue(xd, wq, S), nv.gemm_residue(xd, wt, S)
        z0, z1 = y0, y1
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(z0, z1)


@pytest.mark.parametrize("M,N,K", [(1, 512, 28672), (2, 256, 16384), (8, 700, 4096), (3, 40, 10000 // 16 * 16)])
def test_in_launch_quantization_shapes(nv, orc, M, N, K):
    """Raw activations small enough to be quantized inside the decode launch, including
    K ranges split over workgroups (amax then read separately from the range's chunks):
    the product must match the oracle's on the oracle-quantized operands."""
    x = inputs.small_random(500 + M, M, K)
    w = inputs.small_random(501 + N, N, K, scale=0.02)
    note(f"in-launch quantization M={M} N={N} K={K}")
    wq = nv.quantize(w.to(DEV))
    y = nv.gemm(x.to(DEV), wq)
    torch.cuda.synchronize()
    ref = orc.gemm(orc.quantize(x), orc.quantize(w))
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, err


@pytest.mark.parametrize("M,N,K", [(700, 16400, 1040), (300, 16400, 1040), (520, 12304, 2064), (100, 300, 1040),
                                   (300, 3000, 16400), (520, 8960, 1040)])
def test_prefill_large_tiles_ragged(nv, orc, M, N, K):
    """Shapes that take the pipelined product (256 x 256 and 128 x 128 tiles, and
    256 x 256 with K split four ways): ragged M, N, and a K ending in a half chunk.
    Sampled outputs against the oracle; row-major and tiled weights give identical bits."""
    x = inputs.small_random(800 + M, M, K)
    w = inputs.small_random(801 + N, N, K, scale=0.02)
    note(f"large-tile prefill M={M} N={N} K={K}")
    xd = x.to(DEV)
    wq = nv.quantize(w.to(DEV))
    wt = nv.pack_tiled(wq)
    y = nv.gemm(xd, wq)
    yt = nv.gemm(xd, wt)
    torch.cuda.synchronize()
    assert torch.equal(y, yt)
    rng = np.random.default_rng(M + N)
    ms = np.concatenate([rng.integers(0, M, 1500), [M - 1, M - 1, 0]])
    ns = np.concatenate([rng.integers(0, N, 1500), [N - 1, 0, N - 1]])
    xq = orc.quantize(x)
    rows = np.unique(ns)
    wsub = orc.quantize(w[rows], static_S=float(orc.tensor_scale(w)))
    wpos = {r: i for i, r in enumerate(rows)}
    ref = orc.gemm_pairs(xq, wsub, ms, np.array([wpos[n] for n in ns]))
    err = gemm_error(y.cpu().numpy()[ms, ns], ref)
    assert err <= TOL, err
