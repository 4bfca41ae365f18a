"""Decode attention over an NVFP4 KV cache with the residue on its activation
operands (ResServe abstract: decode attention), GPU against the oracle: the caches
bit for bit, the output within the floored relative error (C16), with and without
compensation, at ragged and at the bench's sizes, and the two closed forms of the
oracle's pins (uniform scores, one dominant token) on the GPU."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_02_amd import inputs
from helpers import assert_qtensor_equal, gemm_error, note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


@pytest.fixture(scope="module")
def nv():
    from block_scaled_fp4_02_amd import nvfp4
    nvfp4.lib()
    return nvfp4


def _run(nv, orc, q, k, vt, H, T, D, comp, q_f32=False):
    note(f"attention H={H} T={T} D={D} compensate={comp} q_f32={q_f32}")
    qd = (q.float() if q_f32 else q).to(DEV)
    kq, vq = nv.quantize(k.to(DEV)), nv.quantize(vt.to(DEV))
    o = nv.decode_attention(qd, kq, vq, T, compensate=comp)
    torch.cuda.synchronize()
    okq, ovq = orc.quantize(k), orc.quantize(vt)
    assert_qtensor_equal(kq, okq, "K cache")
    assert_qtensor_equal(vq, ovq, "V cache")
    ref = orc.decode_attention(q.float().numpy(), okq, ovq, H, T, D, comp)
    return o.cpu().numpy(), ref


@pytest.mark.parametrize("comp", [True, False])
@pytest.mark.parametrize("H,T,D,q_f32", [(4, 256, 64, False), (3, 272, 96, True), (2, 16, 32, False),
                                         (5, 1040, 256, False), (1, 4112, 128, True)])
def test_attention_matches_oracle(nv, orc, H, T, D, q_f32, comp):
    q, k, vt = inputs.attention(H, T, D, sub=H + T + D)
    o, ref = _run(nv, orc, q, k, vt, H, T, D, comp, q_f32)
    err = gemm_error(o, ref)
    assert err <= TOL, err


def test_attention_bench_shape(nv, orc):
    """The bench's 32 heads x 4096 tokens x 128, compensated, all heads."""
    H, T, D = inputs.ATTN_SHAPE
    q, k, vt = inputs.attention(H, T, D)
    o, ref = _run(nv, orc, q, k, vt, H, T, D, True)
    assert gemm_error(o, ref) <= TOL


@pytest.mark.parametrize("comp", [True, False])
def test_attention_closed_forms(nv, orc, comp):
    """Identical K rows give p = 1/T and o = the mean of the dequantized V; one token
    whose score dominates gives p one-hot and o = its V column (to FP32 rounding of the
    probabilities' tensor scale)."""
    H, T, D = 2, 64, 32
    g = np.random.default_rng(11)
    vt = torch.from_numpy(g.standard_normal((H * D, T)).astype(np.float32))
    q = torch.from_numpy(g.standard_normal((H, D)).astype(np.float32))
    k = torch.from_numpy(np.repeat(g.standard_normal((1, D)).astype(np.float32), H * T, axis=0))
    o, _ = _run(nv, orc, q, k, vt, H, T, D, comp, q_f32=True)
    vd = orc.dequantize(orc.quantize(vt)).reshape(H, D, T)
    np.testing.assert_allclose(o, vd.mean(axis=2), rtol=2e-6, atol=1e-6)
    hot = 37
    q = torch.zeros((H, D), dtype=torch.float32)
    q[:, 0] = 64.0
    k = torch.zeros((H * T, D), dtype=torch.float32)
    k[[h * T + hot for h in range(H)], 0] = 64.0
    o, _ = _run(nv, orc, q, k, vt, H, T, D, comp, q_f32=True)
    np.testing.assert_allclose(o, vd[:, :, hot], rtol=2e-6, atol=1e-6)


def test_attention_one_hot_small_scales(nv, orc):
    """One dominant token whose V block is scaled down row by row (factors 2^0 ..
    2^-19), so its E4M3 block scales run from normal through the subnormal codes to
    zero: o equals that token's dequantized V column to FP32 rounding, element by
    element and without an absolute floor (a wrong scale decode at any code shows)."""
    H, T, D = 2, 64, 128
    hot = 21
    g = np.random.default_rng(12)
    vt = g.standard_normal((H * D, T)).astype(np.float32)
    blk = slice(16 * (hot // 16), 16 * (hot // 16) + 16)
    for r in range(H * D):
        vt[r, blk] *= np.float32(2.0 ** -(r % 20))
    vt = torch.from_numpy(vt)
    q = torch.zeros((H, D), dtype=torch.float32)
    q[:, 0] = 64.0
    k = torch.zeros((H * T, D), dtype=torch.float32)
    k[[h * T + hot for h in range(H)], 0] = 64.0
    codes = orc.quantize(vt)
    sb = np.asarray(codes.scales)[:, hot // 16]
    assert ((sb > 0) & (sb < 8)).any() and (sb >= 8).any()      # subnormal and normal codes
    vd = orc.dequantize(codes).reshape(H, D, T)
    for comp in (True, False):
        o, _ = _run(nv, orc, q, k, vt, H, T, D, comp, q_f32=True)
        np.testing.assert_allclose(o, vd[:, :, hot], rtol=2e-6, atol=0)


def test_attention_repeat_and_graph(nv):
    """Deterministic across calls, and a captured graph replays to the same bits."""
    H, T, D = 4, 512, 64
    q, k, vt = inputs.attention(H, T, D, sub=9)
    qd = q.to(DEV)
    kq, vq = nv.quantize(k.to(DEV)), nv.quantize(vt.to(DEV))
    o1 = nv.decode_attention(qd, kq, vq, T)
    o2 = nv.decode_attention(qd, kq, vq, T)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    out = torch.empty_like(o1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        nv.decode_attention(qd, kq, vq, T, out=out)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):
            nv.decode_attention(qd, kq, vq, T, out=out)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        out.zero_()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o1), i
