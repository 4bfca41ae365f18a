"""nvfp4_gemm_noalloc (the entry point that allocates nothing) against nvfp4_gemm,
through the C ABI: the same kernels on the same inputs must give the same bits, on
two calls in a row -- the second with a smaller input, so that state left in the
shared static scratch by the first (quantized activations, split-K partials, the
arrival slots and tile counters) cannot leak into it."""
import pytest
import torch

from block_scaled_fp4_02_amd import inputs
from helpers import note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def nv():
    from block_scaled_fp4_02_amd import nvfp4
    nvfp4.lib()
    return nvfp4


def _pair(nv, M, N, K, seed, tiled, prequant):
    x = inputs.small_random(seed, M, K).to(DEV)
    wq = nv.quantize(inputs.small_random(seed + 1, N, K, scale=0.02).to(DEV))
    if tiled:
        wq = nv.pack_tiled(wq)
    a = nv.quantize(x) if prequant else x
    return a, wq


# (M, N, K): fused decode with in-launch quantization; the separate small quantizer
# and a split-K decode plan; the windowed kernel; the tile path (prefill kernel)
CASES = [((16, 14336, 4096), (4, 300, 1024)),
         ((16, 4096, 14336), (2, 700, 4096)),
         ((64, 2048, 4096), (40, 300, 1040)),
         ((300, 1000, 2048), (130, 300, 528))]


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("prequant", [False, True])
@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_gemm(nv, first, second, tiled, prequant):
    for i, (M, N, K) in enumerate((first, second)):
        note(f"noalloc call {i}: M={M} N={N} K={K} tiled={tiled} prequant={prequant}")
        a, w = _pair(nv, M, N, K, 40 + 7 * i + M, tiled, prequant)
        ref = nv.gemm(a, w)
        got = torch.full_like(ref, float("nan"))
        nv.gemm_noalloc(a, w, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (i, M, N, K)


def test_noalloc_bf16_output_and_repeat(nv):
    a, w = _pair(nv, 8, 6144, 4096, 77, True, False)
    ref = nv.gemm(a, w, out_dtype=torch.bfloat16)
    for i in range(3):
        note(f"noalloc bf16 repeat {i}")
        got = torch.zeros_like(ref)
        nv.gemm_noalloc(a, w, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), i


def test_noalloc_rejects_oversized_workspace(nv):
    """A product whose workspace exceeds the static scratch fails before anything runs."""
    from block_scaled_fp4_02_amd.nvfp4 import NVFP4Error
    M, N, K = 512, 8192, 28672
    need = nv.lib().nvfp4_workspace_size(1, M, N, K, 0)
    assert need > nv.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    w = nv.NVFP4Tensor.empty(N, K, DEV)
    y = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(NVFP4Error) as ei:
        nv.gemm_noalloc(x, w, y)
    assert ei.value.status == 5
    assert b"static scratch" in nv.lib().nvfp4_last_error()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
