"""The whole-batch comparison helper (tests/oracle_pool.py) on the CPU: fed the
oracle's own results it reports zero error for every request, and a planted
difference in one request's results shows up in that request only."""
import numpy as np

import oracle as O
import oracle_pool as P
import workloads as W


def _oracle_results(wl):
    Oo, Uo, _, _ = O.verify_batch(wl.S0, wl.q64(), wl.k64(), wl.v64(), wl.g, wl.beta, wl.node_offset, wl.parent,
                                  wl.Hv, wl.Hk)
    po, plo, _ = O.accepted_path_batch(wl.node_offset, wl.parent, wl.accept_node, max_nodes=64)
    So, _ = O.commit_batch(wl.S0, wl.q64(), wl.k64(), wl.v64(), wl.g, wl.beta, wl.node_offset, wl.parent, po, plo,
                           wl.Hv, wl.Hk)
    return Oo.astype(np.float32), Uo.astype(np.float32), So.astype(np.float32)


def test_pool_reports_every_request_and_finds_a_planted_difference():
    wl = W.make_mixed_b256(per_kind=2, Hv=2, Hk=1, seed=3)
    out, U, S1 = _oracle_results(wl)
    b_bad = 5
    lo = int(wl.node_offset[b_bad])
    out[lo, 1, 7] += 0.5 * np.abs(out[lo, 1]).max()     # a planted error in one request's output
    S1[2, 0, 3, 4] *= -1.0                               # and one in another request's state
    arrays = P.workload_arrays(wl)
    arrays.update(out=out, U=U, S1=S1)
    res = sorted(P.run(arrays, P.verify_commit_request, [(b, wl.Hv, wl.Hk) for b in range(wl.B)]))
    assert [r[0] for r in res] == list(range(wl.B))
    for b, st, eo, eu, es in res:
        assert st == 0 and eu < 1e-6
        assert (eo > 0.1) == (b == b_bad), b
        if b != 2:
            assert es < 1e-6, b
    assert res[2][4] > 1e-3 or wl.S0[2, 0, 3, 4] == 0
