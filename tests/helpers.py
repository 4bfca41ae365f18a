"""Shared helpers for the GPU parity tests (no NVFP4 arithmetic here)."""
import os
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


# every gemm_error comparison of the session: (test, floored error, normwise error,
# floor-clamped elements, elements); conftest prints a summary at the end
P2_RECORDS = []


def gemm_error(y, y_ref) -> float:
    """max |y - y*| / max(|y*|, 1e-3 max|y*|) -- the floored relative error. Also records
    the plain normwise max|y - y*| / max|y*| and how many elements sit below the floor."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return 0.0
    amax = np.max(np.abs(y_ref))
    floor = 1e-3 * amax
    den = np.maximum(np.abs(y_ref), floor if floor > 0 else 1e-30)
    diff = np.abs(y - y_ref)
    err = float(np.max(diff / den))
    normwise = float(np.max(diff) / amax) if amax > 0 else float(np.max(diff))
    clamped = int(np.count_nonzero(np.abs(y_ref) < floor))
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    P2_RECORDS.append((test, err, normwise, clamped, int(y_ref.size)))
    return err


def bf16_bound_ok(y_bf16, y_ref, tol=2e-3) -> bool:
    """|y - y*| <= tol * max(|y*|, floor) + 2^-8 |y*|: half a bf16 ulp on top of the FP32 bar."""
    y = np.asarray(y_bf16, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    floor = 1e-3 * np.max(np.abs(y_ref))
    bound = tol * np.maximum(np.abs(y_ref), floor) + 2.0 ** -8 * np.abs(y_ref)
    return bool(np.all(np.abs(y - y_ref) <= bound))


def untile(codes_t, scales_t, rows: int, K: int):
    """Row-major (codes [rows, K/2], scales [rows, K/16]) of a tiled NVFP4 tensor, and
    whether its padding is zero, following the layout as documented in include/nvfp4.h
    (item (t, u) of 16 rows x 512 columns; byte 1024 i + 16 p + j of its codes is byte j
    of row 16 t + p % 16 from column 512 u + 128 (p // 16) + 32 i; scale byte 8 p + b is
    the block of columns 512 u + 128 (p // 16) + 16 b)."""
    nt, ku = (rows + 15) // 16, (K + 511) // 512
    c = np.asarray(codes_t).reshape(nt, ku, 4, 4, 16, 16)     # t, u, i, g, r, j
    s = np.asarray(scales_t).reshape(nt, ku, 4, 16, 8)        # t, u, g, r, b
    codes = c.transpose(0, 4, 1, 3, 2, 5).reshape(nt * 16, ku * 512 // 2)   # rows, (u, g, i, j)
    scales = s.transpose(0, 3, 1, 2, 4).reshape(nt * 16, ku * 32)          # rows, (u, g, b)
    pad_zero = (not codes[rows:].any() and not codes[:, K // 2:].any() and not scales[rows:].any()
                and not scales[:, K // 16:].any())
    return codes[:rows, :K // 2], scales[:rows, :K // 16], pad_zero
