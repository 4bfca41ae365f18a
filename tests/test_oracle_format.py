"""Pins of the oracle's number formats and rounding against facts fixed outside it.

* E2M1 codebook and E4M3 maximum / step from tests/golden/nvfp4_format.json
  (ARCQuant article on zizhi168.cn, sections 1 and 4.2);
* E4M3 decoding and round-to-nearest-even against torch's float8_e4m3fn
  (an independent library implementation);
* E2M1 round-to-nearest-even against numpy's rint on the scaled grid (a
  different method from the oracle's brute-force nearest search).
"""
import json
import os

import numpy as np
import pytest
import torch

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_format.json")))


def test_e2m1_codebook(orc):
    book = GOLD["e2m1_codebook"]["value"]
    for c in range(8):
        assert orc.e2m1_value(c) == book[c]
        assert orc.e2m1_value(c | 8) == -book[c]
    assert np.signbit(orc.e2m1_value(8))          # code 8 is -0


def test_e4m3_decode_matches_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        v = orc.e4m3_value(b)
        if np.isnan(ref[b]):
            assert np.isnan(v), b
        else:
            assert v == ref[b], b
    assert orc.e4m3_value(0x7E) == GOLD["e4m3_max"]["value"]
    finite = [orc.e4m3_value(b) for b in range(127)]
    assert max(finite) == GOLD["e4m3_max"]["value"]
    # relative step 2^-3 between consecutive normal values
    step = GOLD["e4m3_relative_step"]["value"]
    for b in range(8, 126):
        lo, hi = orc.e4m3_value(b), orc.e4m3_value(b + 1)
        binade = 2.0 ** np.floor(np.log2(lo))
        assert hi - lo == step * binade


def test_e4m3_encode_matches_torch(orc):
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.uniform(0, 448, 4000), 2.0 ** rng.uniform(-14, 8.8, 4000),
        [0.0, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -9, 2.0 ** -6, 448.0, 1.0625, 1.1875, 2.0 ** -6 - 2.0 ** -10],
    ]).astype(np.float32)
    # midpoints between all consecutive finite values (ties must go to the even code)
    finite = np.array([orc.e4m3_value(b) for b in range(127)])
    mids = ((finite[:-1] + finite[1:]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mids])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(v) for v in vals])
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates(orc):
    for v in [448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 1e20, 3e38]:
        assert orc.e4m3_encode(v) == 0x7E


def test_e2m1_encode_saturates_far_above(orc):
    # far above 6 every double distance rounds alike; the result must still be 6
    for q in [6.0, 7.0, 1e9, 1e20, 1e30, 3e38]:
        assert orc.e2m1_encode(q) == 7
        assert orc.e2m1_encode(-q) == 15


def _rint_e2m1(q: np.ndarray) -> np.ndarray:
    """Round |q| to the E2M1 grid with numpy's ties-to-even rint, binade by binade."""
    a = np.abs(q.astype(np.float64))
    out = np.where(a < 2, np.rint(a * 2) / 2, np.where(a < 4, np.rint(a), np.rint(a / 2) * 2))
    return np.minimum(out, 6.0)


def test_e2m1_encode_matches_rint(orc):
    rng = np.random.default_rng(3)
    book = np.array(GOLD["e2m1_codebook"]["value"])
    mids = (book[:-1] + book[1:]) / 2
    q = np.concatenate([rng.uniform(-7, 7, 20000), book, -book, mids, -mids,
                        np.nextafter(mids, 0), np.nextafter(mids, 10), [6.4, 6.5, 7.0, 9.0, 1e9, -1e9]])
    q = q.astype(np.float32)
    got = np.array([orc.e2m1_value(orc.e2m1_encode(v)) for v in q])
    want = _rint_e2m1(q) * np.where(np.signbit(q), -1, 1)
    assert np.array_equal(got, want)


def test_e2m1_ties_from_golden(orc):
    for q, v in GOLD["e2m1_ties"]["value"]:
        assert orc.e2m1_value(orc.e2m1_encode(q)) == v
        assert orc.e2m1_value(orc.e2m1_encode(-q)) == -v


def test_e2m1_sign_of_zero(orc):
    assert orc.e2m1_encode(-0.0) == 8
    assert orc.e2m1_encode(-0.1) == 8
    assert orc.e2m1_encode(0.1) == 0
