"""Host-side checks of bench.py: the one-GPU guard and the committed traffic figure."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 exits with status 2 and says why, before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profiled_traffic_matches_the_algorithmic_bytes():
    """The committed pmc summary of the decode sweep, when it was taken on the current
    decode source, gives HBM bytes per launch no lower than the algorithmic bytes of the
    15 cases (weights, activation and output once each) and at most 20% above them."""
    import bench
    t = bench.profiled_traffic()
    if t is None:
        pytest.skip("the decode source changed since the committed counters were taken")
    cases = [(M, K, N) for (K, N) in ((4096, 14336), (14336, 4096), (4096, 6144)) for M in (1, 2, 4, 8, 16)]
    alg = sum(N * K // 2 + N * K // 16 + M * K // 2 + M * K // 16 + 4 * M * N for M, K, N in cases) / len(cases)
    assert alg <= t <= 1.2 * alg, (t, alg)
