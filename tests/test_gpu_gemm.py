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


LAYOUTS = ["rowmajor", "tiled"]


def _layout(nv, wq, layout):
    """The weight in the layout under test (the bench times the tiled one)."""
    return nv.pack_tiled(wq) if layout == "tiled" else wq


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemv_4096(nv, orc, layout):
    x, w = inputs.gemv_4096()
    note(f"gemm gemv 1x4096x4096 {layout}")
    wq = nv.quantize(w.to(DEV))
    y = nv.gemm(x.to(DEV), _layout(nv, wq, layout))
    torch.cuda.synchronize()
    ow = orc.quantize(w)
    assert_qtensor_equal(wq, ow, "W")
    ref = orc.gemm(orc.quantize(x), ow)
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, err


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("shape_idx", [0, 1, 2])
def test_decode_sweep(nv, orc, shape_idx, layout):
    """Every output of the fused call (activation quantized in the call) and of the
    product on pre-quantized activations (the kernel the bench's roofline times)."""
    K, N = inputs.DECODE_SHAPES[shape_idx]
    x, w = inputs.decode_sweep(shape_idx)
    note(f"gemm decode sweep K={K} N={N} {layout}: quantize W")
    wq = nv.quantize(w.to(DEV))
    torch.cuda.synchronize()
    ow = orc.quantize(w)
    assert_qtensor_equal(wq, ow, "W")
    wl = _layout(nv, wq, layout)
    xd = x.to(DEV)
    for M in inputs.DECODE_MS:
        note(f"gemm decode M={M} K={K} N={N} {layout}")
        y = nv.gemm(xd[:M], wl)
        aq = nv.quantize(xd[:M])
        yk = nv.gemm(aq, wl)
        torch.cuda.synchronize()
        ox = orc.quantize(x[:M])
        assert_qtensor_equal(aq, ox, "X")
        ref = orc.gemm_blas(ox, ow)
        err = gemm_error(y.cpu().numpy(), ref)
        assert err <= TOL, (M, err)
        err = gemm_error(yk.cpu().numpy(), ref)
        assert err <= TOL, (M, "pre-quantized", err)


def test_prequantized_activation_path(nv, orc):
    x, w = inputs.decode_sweep(2)
    wq = nv.quantize(w.to(DEV))
    xq = nv.quantize(x[:8].to(DEV))
    note("gemm with pre-quantized activations")
    y1 = nv.gemm(xq, wq)
    y2 = nv.gemm(x[:8].to(DEV), wq)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.fixture(scope="module")
def residue_case(orc):
    x, w = inputs.residue_8192(16)
    return x, w, orc.quantize(w), orc.weight_aug(w, 8192)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M", inputs.RESIDUE_MS)
def test_residue_k_to_2k(nv, orc, residue_case, M, layout):
    x, w, ow, wa = residue_case
    x = x[:M]
    note(f"gemm_residue K->2K M={M} {layout}")
    wq = _layout(nv, nv.quantize(w.to(DEV)), layout)
    y, aug = nv.gemm_residue(x.to(DEV), wq, 8192, return_aug=True)
    y0 = nv.gemm(x.to(DEV), wq)
    torch.cuda.synchronize()
    xa = orc.quantize_aug(x, S_cols=8192)
    assert_qtensor_equal(aug, xa, "X_aug")
    ref = orc.gemm_blas(xa, wa)
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, err
    # the compensated product is closer to the product with unquantized activations
    exact = x.float().numpy().astype(np.float64) @ orc.dequantize(ow).T
    e_res = np.linalg.norm(y.cpu().numpy() - exact)
    e_base = np.linalg.norm(y0.cpu().numpy() - exact)
    assert e_res <= 0.25 * e_base, (e_res, e_base)


@pytest.fixture(scope="module")
def aug_case(orc):
    x, g, xcal, w = inputs.outlier_aug()
    perm = orc.calibrate_perm(xcal, g)
    w_perm = w[:, torch.from_numpy(perm).long()]
    return x, g, perm, w_perm, orc.quantize(w_perm)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("S", inputs.AUG_S)
def test_outlier_augmented(nv, orc, aug_case, S, layout):
    """RMSNorm + calibrated reorder + residue of the top S channels, M=64, N=14336:
    X_aug bit for bit, every output against the oracle."""
    x, g, perm, w_perm, ow = aug_case
    pd = torch.from_numpy(perm).to(DEV)
    note(f"gemm_residue augmented S={S} {layout}")
    wq = _layout(nv, nv.quantize(w_perm.to(DEV)), layout)
    y, aug = nv.gemm_residue(x.to(DEV), wq, S, gamma=g.to(DEV), eps=1e-6, perm=pd, return_aug=True)
    torch.cuda.synchronize()
    xa = orc.quantize_aug(x, gamma=g, eps=1e-6, perm=perm, S_cols=S)
    assert_qtensor_equal(aug, xa, "X_aug")
    # W_aug = [W' | W'[:, :S]]: its tail codes and scales are the head's
    K = 4096
    wa = orc.QTensor(np.ascontiguousarray(np.concatenate([ow.codes, ow.codes[:, :S // 2]], axis=1)),
                     np.ascontiguousarray(np.concatenate([ow.scales, ow.scales[:, :S // 16]], axis=1)), ow.S, K + S)
    ref = orc.gemm_blas(xa, wa)
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, err


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K,S", [(4, 300, 1024, 256), (12, 300, 1024, 256), (24, 300, 1024, 256),
                                     (8, 14336, 4096, 256), (16, 4096, 14336, 512), (1, 8192, 8192, 2048),
                                     (48, 700, 2048, 512), (16, 1000, 4096, 2048)])
def test_residue_partial_columns(nv, orc, M, N, K, S, layout):
    """Residue columns over a part of K (0 < S < K, K a multiple of 32): the decode
    paths with a separate residue operand, the stacked rows with S < K, the two-row-tile
    instance and the windowed kernel. Every output against the oracle."""
    x = inputs.small_random(300 + M + S, M, K)
    w = inputs.small_random(301 + N, N, K, scale=0.02)
    note(f"gemm_residue partial M={M} N={N} K={K} S={S} {layout}")
    wq = _layout(nv, nv.quantize(w.to(DEV)), layout)
    y, aug = nv.gemm_residue(x.to(DEV), wq, S, return_aug=True)
    torch.cuda.synchronize()
    xa = orc.quantize_aug(x, S_cols=S)
    assert_qtensor_equal(aug, xa, "X_aug")
    ref = orc.gemm_blas(xa, orc.weight_aug(w, S))
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, (err, M, N, K, S)


def _tile_lines(n: int, rng) -> np.ndarray:
    """Indices below n covering every 128- and 256-wide tile of the prefill plans: both
    edges of each 128 band and one interior index per band."""
    idx = []
    for b in range(0, n, 128):
        hi = min(b + 128, n) - 1
        idx += [b, hi, int(rng.integers(b, hi + 1))]
    return np.unique(np.array(idx, dtype=np.int64))


@pytest.fixture(scope="module")
def prefill_case(orc):
    cache = {}

    def get(shape_idx):
        if shape_idx not in cache:
            cache.clear()
            xall, w = inputs.prefill(shape_idx, 8192)
            cache[shape_idx] = (xall, w, orc.tensor_scale(w))
        return cache[shape_idx]
    return get


@pytest.mark.parametrize("M", inputs.PREFILL_MS)
@pytest.mark.parametrize("shape_idx", [0, 1])
def test_prefill_tiles(nv, orc, prefill_case, shape_idx, M):
    """Prefill products at the bench's sizes (tiled weights, as timed): the outputs at
    every output tile's four corners and an interior point, plus 128 random rows and
    columns -- the whole cross product of the chosen rows and columns -- against the
    oracle, for the FP32 accumulator (P2) and the bf16 store of the fused call (half a
    bf16 ulp more). Quantized activations are compared bit for bit: every code at the
    sizes where the oracle quantizes the whole tensor in seconds, else the chosen rows."""
    K, N = inputs.PREFILL_SHAPES[shape_idx]
    xall, w, ow_S = prefill_case(shape_idx)
    rng = np.random.default_rng(1000 * shape_idx + M)
    note(f"prefill K={K} N={N} M={M}: quantize W, tile")
    wq = nv.quantize(w.to(DEV))
    wt = nv.pack_tiled(wq)
    torch.cuda.synchronize()
    assert float(wq.scale.cpu()[0]) == ow_S
    xd = xall[:M].to(DEV)
    note(f"prefill gemm K={K} N={N} M={M}")
    aq = nv.quantize(xd)
    y32 = nv.gemm(aq, wt, out_dtype=torch.float32)
    yb = nv.gemm(xd, wt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([_tile_lines(M, rng), rng.integers(0, M, 128)]))
    cols = np.unique(np.concatenate([_tile_lines(N, rng), rng.integers(0, N, 128)]))
    S_x = orc.tensor_scale(xall[:M])
    assert float(aq.scale.cpu()[0]) == S_x
    ac, as_, _ = aq.host()
    if M * K <= 2048 * 8192:
        ox = orc.quantize(xall[:M])
        assert np.array_equal(ac, ox.codes) and np.array_equal(as_, ox.scales), "X codes differ"
        xq = orc.QTensor(np.ascontiguousarray(ox.codes[rows]), np.ascontiguousarray(ox.scales[rows]), ox.S, K)
    else:
        xq = orc.quantize(xall[rows], static_S=float(S_x))
        assert np.array_equal(ac[rows], xq.codes) and np.array_equal(as_[rows], xq.scales), "X codes differ"
    wsub = orc.quantize(w[cols], static_S=float(ow_S))
    wc, ws_, _ = wq.host()
    assert np.array_equal(wc[cols], wsub.codes) and np.array_equal(ws_[cols], wsub.scales), "W codes differ"
    ref = orc.gemm_blas(xq, wsub)
    got32 = y32.cpu().numpy()[np.ix_(rows, cols)]
    err = gemm_error(got32, ref)
    assert err <= TOL, (M, err)
    gotb = yb.float().cpu().numpy()[np.ix_(rows, cols)]
    assert bf16_bound_ok(gotb, ref), (M, gemm_error(gotb, ref))


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
                                   (300, 3000, 16400), (520, 8960, 1040), (300, 3000, 16416), (700, 1040, 20000)])
def test_prefill_large_tiles_ragged(nv, orc, M, N, K):
    """Shapes that take the pipelined products (256 x 256 and 128 x 128 tiles, and
    256 x 256 with K split four ways; FP4 operands in LDS at K >= 16384 with K a
    multiple of 32): ragged M, N, a K ending in a half chunk, and K ending one or
    few chunks into a 128-column step. Sampled outputs against the oracle; row-major
    and tiled weights give identical bits."""
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


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,S", [(64, 256), (8, 0), (300, 128)])
def test_smoothed_product(nv, orc, aug_case, M, S, layout):
    """Runtime diagonal smoothing with its inverse folded into the weight (OSFP4 abstract):
    Y = Q(smooth(RMSNorm(X))[:, perm]) Q((W diag(1/s))[:, perm])^T, with residue columns;
    every output against the oracle, X_aug bit for bit."""
    x, g, perm, w_perm, _ = aug_case
    K = 4096
    if M > x.shape[0]:
        x = inputs.activations(4, 1, M, K, 0.01, 50.0)
    else:
        x = x[:M]
    sm = np.random.default_rng(M + S).uniform(0.5, 2.0, K).astype(np.float32)
    w = inputs.weights(4, 0, 14336, K, 0.02)
    ws = (w.float() / torch.from_numpy(sm)[None, :]).to(torch.bfloat16)   # the inverse, folded offline
    ws_perm = ws[:, torch.from_numpy(perm).long()]
    note(f"smoothed product M={M} S={S} {layout}")
    wq = _layout(nv, nv.quantize(ws_perm.to(DEV)), layout)
    y, aug = nv.gemm_residue(x.to(DEV), wq, S, gamma=g.to(DEV), eps=1e-6, perm=torch.from_numpy(perm).to(DEV),
                             smooth=torch.from_numpy(sm).to(DEV), return_aug=True)
    torch.cuda.synchronize()
    xa = orc.quantize_aug(x, gamma=g, eps=1e-6, perm=perm, S_cols=S, smooth=sm)
    assert_qtensor_equal(aug, xa, "X_aug")
    ref = orc.gemm_blas(xa, orc.weight_aug(ws_perm, S))
    err = gemm_error(y.cpu().numpy(), ref)
    assert err <= TOL, err


def _waug(q, S):
    """W_aug = [W' | W'[:, :S]] from the quantized W': the tail's codes and block scales
    are the head's (same blocks, same tensor scale)."""
    import oracle
    return oracle.QTensor(np.ascontiguousarray(np.concatenate([q.codes, q.codes[:, :S // 2]], axis=1)),
                          np.ascontiguousarray(np.concatenate([q.scales, q.scales[:, :S // 16]], axis=1)),
                          q.S, q.K + S)


@pytest.mark.parametrize("M,N,K,S,layouts", [(520, 3000, 4096, 256, LAYOUTS), (2048, 28672, 8192, 512, ["tiled"]),
                                             (512, 8192, 28672, 1024, ["tiled"]), (300, 1000, 2048, 2048, LAYOUTS)])
def test_prefill_selective_residue(nv, orc, M, N, K, S, layouts):
    """Selective compensation at prompt sizes (ResServe abstract; ARCQuant article, sections
    3.1-3.2): RMSNorm, calibrated reorder and the residue of the top S channels, in the
    pipelined matrix-core product (split K at 512 x 8192 x 28672). X_aug bit for bit; the
    outputs at every tile's corners and an interior point against the oracle."""
    rng = np.random.default_rng(M + S)
    x = inputs.activations(5, 2, M, K, 0.01, 50.0)
    g = inputs.gamma(5, 2, K)
    xcal = inputs.activations(5, 2, 512, K, 0.01, 50.0, tensor=inputs.T_XCAL)
    perm = orc.calibrate_perm(xcal, g)
    w = inputs.weights(5, 2, N, K, 0.015)[:, torch.from_numpy(perm).long()]
    note(f"prefill selective residue M={M} N={N} K={K} S={S}: quantize")
    wq = nv.quantize(w.to(DEV))
    pd = torch.from_numpy(perm).to(DEV)
    xa = orc.quantize_aug(x, gamma=g, eps=1e-6, perm=perm, S_cols=S)
    rows = np.unique(np.concatenate([_tile_lines(M, rng), rng.integers(0, M, 64)]))
    cols = np.unique(np.concatenate([_tile_lines(N, rng), rng.integers(0, N, 64)]))
    S_w = orc.tensor_scale(w)
    wsub = _waug(orc.quantize(w[cols], static_S=float(S_w)), S)
    xsub = orc.QTensor(np.ascontiguousarray(xa.codes[rows]), np.ascontiguousarray(xa.scales[rows]), xa.S, K + S)
    ref = orc.gemm_blas(xsub, wsub)
    for layout in layouts:
        note(f"prefill selective residue M={M} N={N} K={K} S={S} {layout}")
        wl = _layout(nv, wq, layout)
        y, aug = nv.gemm_residue(x.to(DEV), wl, S, gamma=g.to(DEV), eps=1e-6, perm=pd, return_aug=True)
        yb = nv.gemm_residue(x.to(DEV), wl, S, gamma=g.to(DEV), eps=1e-6, perm=pd, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert_qtensor_equal(aug, xa, "X_aug")
        err = gemm_error(y.cpu().numpy()[np.ix_(rows, cols)], ref)
        assert err <= TOL, (err, layout)
        assert bf16_bound_ok(yb.float().cpu().numpy()[np.ix_(rows, cols)], ref), layout
