"""Whole-batch comparison of device results with the fp64 oracle, over a process pool.

Test infrastructure only.  The parent writes a workload's arrays and the device's
results into a temporary directory as .npy files; each worker process memory-maps
them and evaluates the oracle for one request at a time, returning that request's
worst row-normwise relative errors.  Nothing here computes a result the oracle
does not: the workers call oracle functions and measure differences.

The pool has one process per host core, at most 16 (the host share that comes
with one GPU), and uses the spawn start method: the parent may already hold a
GPU context, and the workers never touch the GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import sys
import tempfile
import time

import numpy as np

_D = {}      # worker side: memory-mapped arrays by name
_W = {}      # worker side: widened (float64) copies, made once per worker


def pool_size() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _init(dirname, names):
    os.environ["OMP_NUM_THREADS"] = "1"
    for n in names:
        _D[n] = np.load(os.path.join(dirname, n + ".npy"), mmap_mode="r")


_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def run(arrays: dict, fn, items, label: str = ""):
    """fn(item) for every item, in worker processes that see `arrays` (by name) as _D.

    Each worker's BLAS runs single-threaded (the variables are set before the
    workers start, so numpy sees them at import): one process per core is the
    parallelism.  A progress line goes to the process's real stderr every ~20 s,
    past any output capture, so a long comparison is visibly alive."""
    items = list(items)
    tmp = tempfile.mkdtemp(prefix="gdn_oracle_pool_")
    saved = {k: os.environ.get(k) for k in _THREAD_VARS}
    try:
        for name, arr in arrays.items():
            np.save(os.path.join(tmp, name + ".npy"), np.ascontiguousarray(arr))
        for k in _THREAD_VARS:
            os.environ[k] = "1"
        ctx = mp.get_context("spawn")
        out, t0 = [], time.time()
        last = t0
        with ctx.Pool(pool_size(), initializer=_init, initargs=(tmp, list(arrays))) as pool:
            for r in pool.imap_unordered(fn, items, chunksize=1):
                out.append(r)
                if time.time() - last > 20:
                    last = time.time()
                    print(f"[oracle pool {label}] {len(out)}/{len(items)} done in {last - t0:.0f} s",
                          file=sys.__stderr__, flush=True)
        return out
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        shutil.rmtree(tmp, ignore_errors=True)


def _wide(name):
    """bf16 bit patterns (uint16) of _D[name] widened exactly to float64, once per worker."""
    if name not in _W:
        import workloads as W
        a = _D[name]
        _W[name] = W.bf16_bits_to_f32(np.asarray(a)).astype(np.float64) if a.dtype == np.uint16 else \
            np.asarray(a, np.float64)
    return _W[name]


def rowwise(x, ref):
    """max over rows (last axis) of ||x - ref||_inf / ||ref||_inf; rows of ref that are
    exactly zero must be exactly zero in x."""
    x = np.asarray(x, np.float64).reshape(-1, np.shape(x)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.abs(x - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    if not np.all(np.isfinite(num)):
        return float("inf")
    zero = den == 0
    if zero.any() and not np.all(num[zero] == 0):
        return float("inf")
    return float((num[~zero] / den[~zero]).max()) if (~zero).any() else 0.0


def _unit_inputs(prefix, b, Hv, Hk, S0=None, slot=None):
    import oracle as O
    off, par = _D[prefix + "node_offset"], _D[prefix + "parent"]
    S = _D[prefix + "S0"] if S0 is None else S0
    return O.verify_request(S, _wide(prefix + "q"), _wide(prefix + "k"), _wide(prefix + "v"),
                            np.asarray(_D[prefix + "g"]), np.asarray(_D[prefix + "beta"]), off, par, b, Hv, Hk,
                            max_nodes=int(_D[prefix + "max_nodes"]),
                            state_slot=None if slot is None else np.full(len(off) - 1, slot, np.int32))


def verify_commit_request(task):
    """Request b of one tree: the oracle's outputs, pseudo-values and committed state
    (along the request's accepted node) against the device's out, U and S1.
    Returns (b, status, err_out, err_U, err_S)."""
    import oracle as O
    b, Hv, Hk = task
    st, Ob, Ub, _, states = _unit_inputs("", b, Hv, Hk)
    if st != O.STATUS_OK:
        return b, st, 0.0, 0.0, 0.0
    lo, hi = int(_D["node_offset"][b]), int(_D["node_offset"][b + 1])
    eo = rowwise(_D["out"][lo:hi], Ob) if hi > lo else 0.0
    eu = rowwise(_D["U"][lo:hi], Ub) if hi > lo else 0.0
    path = O.accepted_path(_D["parent"][lo:hi], int(_D["accept_node"][b]))
    es = 0.0
    for h in range(Hv):
        want = O.commit_unit(_D["S0"][b, h], states[h], path)
        es = max(es, rowwise(np.asarray(_D["S1"][b, h]).reshape(1, -1), want.reshape(1, -1)))
    return b, st, eo, eu, es


def commit_then_verify_request(task):
    """Request b of a decoding step: commit the previous tree (prefix P_) along its accepted
    node, then verify the next tree (prefix C_) from that state, all in the oracle; against
    the device's S_f, out_f and U_f.  Returns (b, err_S, err_out, err_U)."""
    import oracle as O
    b, Hv, Hk = task
    st, _, _, _, states = _unit_inputs("P_", b, Hv, Hk)
    assert st == O.STATUS_OK
    plo, phi = int(_D["P_node_offset"][b]), int(_D["P_node_offset"][b + 1])
    path = O.accepted_path(_D["P_parent"][plo:phi], int(_D["P_accept_node"][b]))
    S_mid = np.stack([O.commit_unit(_D["P_S0"][b, h], states[h], path) for h in range(Hv)])
    es = rowwise(np.asarray(_D["S_f"][b]).reshape(Hv, -1), S_mid.reshape(Hv, -1))
    st2, Ob, Ub, _, _ = _unit_inputs("C_", b, Hv, Hk, S0=S_mid[None], slot=0)
    assert st2 == O.STATUS_OK
    lo, hi = int(_D["C_node_offset"][b]), int(_D["C_node_offset"][b + 1])
    eo = rowwise(_D["out_f"][lo:hi], Ob) if hi > lo else 0.0
    eu = rowwise(_D["U_f"][lo:hi], Ub) if hi > lo else 0.0
    return b, es, eo, eu


def attention_request(b):
    """Request b of a tree-attention batch: the oracle's rows against every device result
    named out_<i> / lse_<i>.  Returns (b, [(err_out, err_lse) per result])."""
    from oracle import tree_attention as A
    import workloads as W
    f = lambda x: W.bf16_bits_to_f32(np.asarray(x)).astype(np.float64)
    lo, hi = int(_D["node_offset"][b]), int(_D["node_offset"][b + 1])
    c0, c1 = int(_D["ctx_offset"][b]), int(_D["ctx_offset"][b + 1])
    if hi == lo:
        return b, []
    ro, rl = A.tree_attention_request(f(_D["q"][lo:hi]), f(_D["k_ctx"][c0:c1]), f(_D["v_ctx"][c0:c1]),
                                      f(_D["k_node"][lo:hi]), f(_D["v_node"][lo:hi]), _D["parent"][lo:hi],
                                      float(_D["scale"]))
    errs = []
    i = 0
    while f"out_{i}" in _D:
        eo = rowwise(_D[f"out_{i}"][lo:hi], ro)
        el = float(np.abs(np.asarray(_D[f"lse_{i}"][lo:hi], np.float64) - rl).max())
        errs.append((eo, el if np.isfinite(el) else float("inf")))
        i += 1
    return b, errs


def workload_arrays(wl, prefix=""):
    """The arrays of a verify workload the workers read, under prefix."""
    return {prefix + "S0": wl.S0, prefix + "q": wl.q, prefix + "k": wl.k, prefix + "v": wl.v,
            prefix + "g": wl.g, prefix + "beta": wl.beta, prefix + "node_offset": wl.node_offset,
            prefix + "parent": wl.parent, prefix + "accept_node": wl.accept_node,
            prefix + "max_nodes": np.int32(max(1, wl.max_nodes))}
