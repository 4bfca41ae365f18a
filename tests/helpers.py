"""Shared helpers for the GPU parity tests (no NVFP4 arithmetic here)."""
import sys

import numpy as np


def note(msg: str):
    """Name the case before each GPU step, flushed, so a failing run says where it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def assert_qtensor_equal(gpu_t, ref, what: str):
    """Bit-exact comparison of a device NVFP4Tensor against an oracle QTensor."""
    codes, scales, S = gpu_t.host()
    assert S == ref.S, f"{what}: tensor scale {S!r} != {ref.S!r}"
    if not np.array_equal(scales, ref.scales):
        bad = np.argwhere(scales != ref.scales)
        r, b = bad[0]
        raise AssertionError(f"{what}: {len(bad)} block scales differ, first row {r} block {b}: "
                             f"{scales[r, b]:#x} != {ref.scales[r, b]:#x}")
    if not np.array_equal(codes, ref.codes):
        bad = np.argwhere(codes != ref.codes)
        r, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first row {r} byte {j}: "
                             f"{codes[r, j]:#x} != {ref.codes[r, j]:#x}")


def gemm_error(y, y_ref) -> float:
    """max |y - y*| / max(|y*|, 1e-3 max|y*|) -- the floored relative error."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return 0.0
    floor = 1e-3 * np.max(np.abs(y_ref))
    den = np.maximum(np.abs(y_ref), floor if floor > 0 else 1e-30)
    return float(np.max(np.abs(y - y_ref) / den))


def bf16_bound_ok(y_bf16, y_ref, tol=2e-3) -> bool:
    """|y - y*| <= tol * max(|y*|, floor) + 2^-8 |y*|: half a bf16 ulp on top of the FP32 bar."""
    y = np.asarray(y_bf16, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    floor = 1e-3 * np.max(np.abs(y_ref))
    bound = tol * np.maximum(np.abs(y_ref), floor) + 2.0 ** -8 * np.abs(y_ref)
    return bool(np.all(np.abs(y - y_ref) <= bound))
