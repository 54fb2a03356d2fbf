"""bench.py on the host: the multi-GPU refusal and the FLOP accounting of its
headline metric (4 x 128 per visible (query, key) pair, the diagonal chunk
counted causally), checked against a brute-force count over the oracle's
token mask."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import dhsa_oracle as orc  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kept_tile_flops_counts_visible_pairs():
    rng = np.random.default_rng(11)
    hq = 3
    offsets = [np.array([0, 5, 6, 14, 20, 33, 40]), np.array([0, 9, 10, 25])]
    rows = []
    for o in offsets:
        C = len(o) - 1
        per_head = []
        for _h in range(hq):
            per_head.append([sorted(set(rng.choice(i + 1, size=min(i + 1, 3), replace=False)) |
                                    ({i} if rng.random() < 0.8 else set()))
                             for i in range(C)])
        rows.append(per_head)
    rp, ci = orc.rows_to_csr(rows)
    want = 0
    for o, per_head in zip(offsets, rows):
        for h in range(hq):
            want += int(orc.token_mask(o, per_head[h]).sum())
    assert bench.kept_tile_flops(offsets, rp, ci, hq) == 4 * 128 * want
