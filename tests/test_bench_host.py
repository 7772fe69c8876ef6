"""Host-side helpers of bench.py (no GPU): the locality figure it reports
from GPU selections must agree with the oracle's definition."""
import numpy as np

import bench
from oracle import nosa_oracle as O


def test_locality_matches_oracle_definition():
    rng = np.random.default_rng(3)
    steps, units, k = 6, 5, 8
    sels = np.full((steps, units, k), -1, np.int32)
    nsel = np.zeros((steps, units), np.int32)
    blocks = [40, 40, 41, 41, 41, 42]
    for t in range(steps):
        for u in range(units):
            n = int(rng.integers(0, k + 1)) if u else k
            ids = np.sort(rng.choice(blocks[t], size=n, replace=False))
            sels[t, u, :n] = ids
            nsel[t, u] = n
    ref = []
    for t in range(1, steps):
        for u in range(units):
            if nsel[t, u]:
                ref.append(O.locality(list(sels[t - 1, u, : nsel[t - 1, u]]), blocks[t - 1],
                                      list(sels[t, u, : nsel[t, u]])))
    got = bench._locality(list(sels), list(nsel), blocks)
    assert abs(got - float(np.mean(ref))) < 1e-12


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    """The path runs on one GPU: --gpus above 1 ends with status 2 and one
    JSON line saying so, without touching a GPU (this runs on the CPU)."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=root)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "single GPU" in line["error"]


def test_readmissions_match_oracle_definition():
    """The re-admission count bench.py reports from GPU selections agrees with
    the oracle's on random part sequences, and on the oracle's fill trace of a
    small decode run, where it is known to be positive."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        steps = int(rng.integers(1, 9))
        parts = [sorted(rng.choice(12, size=int(rng.integers(0, 6)), replace=False).tolist()) for _ in range(steps)]
        assert bench._readmissions([set(p) for p in parts]) == O.readmissions(parts)
    E = np.float32([10, 9, 8, 7])
    picks = [0, 3, 0]          # the query-aware pick per step, kq = 1, ke = 2
    parts = []
    for p in picks:
        s_q = np.full(4, -1.0, np.float32)
        s_q[p] = 1.0
        g_q, g_f, _ = O.select_blocks_fill(s_q, E, 4, 1, 2)
        parts.append(g_f)
    assert O.readmissions(parts) == bench._readmissions([set(p) for p in parts]) == 1
