"""Algorithmic byte and flop accounting used for the roofline (host logic only)."""
import numpy as np

import bench
import workloads as W


def test_c4_verify_bytes_match_closed_form():
    wl = W.make_custom([W.chain(32)] * 4, [0] * 4, Hv=32, Hk=16, d=4)
    # per request: Hv*(64 KiB + N*1288) + Hk*N*512, plus masks/parents/offsets/status
    per = 32 * (65536 + 32 * 1288) + 16 * 32 * 512
    assert bench.verify_bytes(wl) == 4 * per + wl.T * 12 + 4 * 5 + 4 * 4
    # 1544 B per node-head at r = 2 besides the state
    assert (per - 32 * 65536) / (32 * 32) == 1544


def test_commit_bytes_closed_form():
    wl = W.make_custom([W.chain(3)] * 2, [2, -1], Hv=32, Hk=16, d=4)
    L = np.array([3, 0])
    want = 2 * 32 * 2 * 65536 + 3 * (32 * 516 + 16 * 256) + 4 * 3 + 4 * 2 + 4 * 3
    assert bench.commit_bytes(wl, L) == want


def test_verify_flops_chain():
    wl = W.make_custom([W.chain(3)], [0], Hv=2, Hk=1, d=4)
    # 4 N d^2 + 4 d sum(2 depth - 1) per head, depths 1, 2, 3
    assert bench.verify_flops(wl) == 2 * (4 * 3 * 128 * 128 + 4 * 128 * (1 + 3 + 5))


def test_gpus_above_one_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
