#!/usr/bin/env python3
"""Throughput of tree-structured GDN speculative verify + commit on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixed_b256|random32_b256]

One step = the whole hot path over one batch, as a decoding loop runs it:
gdn_tree_commit_verify commits the previous tree's accepted node into the
state and verifies the next tree (outputs and pseudo-values of every draft
node) from that state in one launch, which reads each state once.  The batch
plays both trees (out of place, so every step is identical).  The same work
as two launches per step, gdn_tree_verify then gdn_tree_commit_node (the
accepted node's root-first path, written out, and the accepted path's
state), is timed first and reported under separate_step; with the path and
the commit as two more launches (gdn_tree_accepted_path, gdn_tree_commit)
under next_rows.  Inputs
are seeded synthetic tensors already resident in HBM; three independent copies
of every buffer are rotated so that no step finds the previous step's data in
the 256 MB Infinity Cache.  Prints ONE JSON line on stdout.

The default workload is the ragged batch-256 mix (64 each of depth-3 chains,
6-node root-branch trees, random 16- and 64-node trees; 48 v-heads, 16 k-heads,
d = 128).  ``value`` is verified tree-nodes per second (a node counts once all
48 heads have verified it; commits/s and node-heads/s ride along).  Per-kernel
durations come from HIP events recorded on the launch stream around every
launch: for the headline step inside the timed region itself (one event per
step boundary), for the two-launch step in a second pass over the same steps.
The snapshot-per-node (storeall) pair is timed
after the main loop for comparison, and the fp64 oracle is timed on a bounded
sample on the host cores.  The rows beyond the core step (acceptance, replay,
budget, tree attention, batch one) are under next_rows, and the other
workloads (depth-3 chains at batch 64, root-branch trees at batch 16 and 1,
random 32-node trees at batch 256) under configs, each launched from Python and
replayed from a HIP graph.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "verified tree-nodes/s (all heads) + commits/s at batch 256; % HBM peak"
D = 128
KERNEL_SOURCES = ("speculative_decoding_tree_amd/csrc/common.h", "speculative_decoding_tree_amd/csrc/mfma.h",
                  "speculative_decoding_tree_amd/csrc/verify.hip", "speculative_decoding_tree_amd/csrc/commit.hip",
                  "speculative_decoding_tree_amd/csrc/attention.hip")


def kernel_source_sha() -> str:
    """sha256 over the sources of the verify and commit kernels."""
    import hashlib
    hsh = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size),
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_sha():
        return None
    key = f"{kernel}.hbm_bytes_per_launch"
    return int(float(vals[key])) if key in vals else None


# ----------------------------------------------------------------------------
# algorithmic bytes (what the method must move, each byte once)
# ----------------------------------------------------------------------------

def verify_bytes(wl) -> int:
    """H0 once per (request, v-head); per node and v-head v (256 B), g and beta
    (8 B), out and U (512 B each); per node and key head q and k (512 B);
    ancestry masks, parents, offsets and statuses."""
    import numpy as np
    n = np.diff(wl.node_offset).astype(np.int64)
    per_req = wl.Hv * (D * D * 4 + n * (2 * D + 8 + 4 * D + 4 * D)) + wl.Hk * n * (4 * D)
    return int(per_req.sum() + wl.T * (8 + 4) + 4 * (wl.B + 1) + 4 * wl.B)


def commit_bytes(wl, path_len) -> int:
    """H0 in and H' out once per (request, v-head); per path node and v-head
    its U row (512 B) and g (4 B); per path node and key head its k row (256 B);
    the path rows."""
    import numpy as np
    L = np.asarray(path_len, np.int64)
    per_req = wl.Hv * (2 * D * D * 4 + L * (4 * D + 4)) + wl.Hk * L * (2 * D)
    return int(per_req.sum() + 4 * L.sum() + 4 * wl.B + 4 * (wl.B + 1))


def verify_flops(wl) -> int:
    """State products 4 N d^2 per unit plus the masked grams and solve/output terms."""
    total = 0
    for b in range(wl.B):
        par = wl.parents_of(b)
        dep = [0] * len(par)
        for i, p in enumerate(par):
            dep[i] = 1 if p < 0 else dep[p] + 1
        n = len(par)
        total += wl.Hv * (4 * n * D * D + 4 * D * sum(2 * x - 1 for x in dep))
    return total


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample, one process per core
# ----------------------------------------------------------------------------

def _oracle_request(args):
    """Worker: verify one request (all heads) and commit its accepted path."""
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import numpy as np
    import oracle as O
    S0, q, k, v, g, beta, parent, accept, Hv, Hk = args
    off = np.array([0, len(parent)], np.int32)
    st, Ob, Ub, anc, states = O.verify_request(S0[None], q, k, v, g, beta, off, parent, 0, Hv, Hk)
    path = O.accepted_path(parent, int(accept))
    for h in range(Hv):
        O.commit_unit(S0[h], states[h], path)
    return len(parent)


def cpu_baseline(wl, n_req: int, min_seconds: float = 10.0, one_core_seconds: float = 4.0):
    """The oracle on the host cores: the first n_req requests, repeated whole
    until at least min_seconds of work have run, one process per core; then the
    same work in this process alone (one core) for about one_core_seconds.

    The pool takes every core this process may run on, at most 16: a host that
    carries one GPU gives it a share of 16 cores, whatever the affinity mask
    shows (the mask is reported beside it)."""
    import multiprocessing as mp
    import numpy as np
    avail = len(os.sched_getaffinity(0))
    cores = min(16, avail)
    q, k, v = wl.q64(), wl.k64(), wl.v64()
    jobs = []
    for b in range(min(n_req, wl.B)):
        lo, hi = wl.node_offset[b], wl.node_offset[b + 1]
        jobs.append((wl.S0[b], q[lo:hi], k[lo:hi], v[lo:hi], wl.g[lo:hi], wl.beta[lo:hi],
                     wl.parent[lo:hi].copy(), wl.accept_node[b], wl.Hv, wl.Hk))
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_request, jobs[:cores])        # warm the workers
        t0 = time.perf_counter()
        nodes, passes = 0, 0
        while passes == 0 or time.perf_counter() - t0 < min_seconds:
            nodes += sum(pool.map(_oracle_request, jobs, chunksize=1))
            passes += 1
        dt = time.perf_counter() - t0
    # one core: the same requests in order, in this process
    t1 = time.perf_counter()
    n1, i = 0, 0
    while i == 0 or time.perf_counter() - t1 < one_core_seconds:
        n1 += _oracle_request(jobs[i % len(jobs)])
        i += 1
    dt1 = time.perf_counter() - t1
    return {"value": nodes / dt, "unit": "nodes/s", "cores": cores, "kind": "oracle",
            "sample": f"first {len(jobs)} of {wl.B} requests of the {wl.name} batch, {passes} passes "
                      f"({nodes} nodes, all {wl.Hv} heads), fp64 verify + commit, one process per core",
            "seconds": dt, "cores_in_affinity_mask": avail,
            "one_core": {"value": n1 / dt1, "unit": "nodes/s", "requests": i, "nodes": n1, "seconds": dt1}}


# ----------------------------------------------------------------------------
# GPU timing
# ----------------------------------------------------------------------------

def _time_launches(fn, n, stream):
    """Average duration (us) of fn() from HIP events recorded around each call."""
    import numpy as np
    import torch
    for _ in range(3):
        fn(0)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3)


def next_rows(args, wl, pools, mn, stream):
    """Rows beyond the core step: device-side greedy acceptance, alone and fused
    with the commit, on the same batch (synthetic draft/target token ids)."""
    import numpy as np
    import torch
    import workloads as W
    from speculative_decoding_tree_amd import gdn_tree as G
    dev = pools[0]["S0"].device
    draft, tgt, root = W.greedy_tokens(wl)
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    dt, tg, rt = tt(draft), tt(tgt), tt(root)
    B = wl.B
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    path = torch.empty((B, mn), dtype=torch.int32, device=dev)
    plen = torch.empty((B,), dtype=torch.int32, device=dev)
    st = torch.empty((B,), dtype=torch.int32, device=dev)
    n = max(10, args.steps // 2)

    def greedy(i):
        p = pools[i % len(pools)]
        G.accept_greedy(p["off"], p["par"], dt, tg, rt, max_nodes=mn, accept_node=acc, path=path,
                        path_len=plen, status=st, stream=stream)

    def fused(i):
        p = pools[i % len(pools)]
        G.accept_commit(p["S0"], p["U"], p["k"], p["g"], p["off"], p["par"], dt, tg, rt, max_nodes=mn,
                        S_out=p["S_out"], accept_node=acc, path=path, path_len=plen, status=st, stream=stream)

    def path_only(i):
        p = pools[i % len(pools)]
        G.accepted_path(p["off"], p["par"], p["acc"], max_nodes=mn, path=path, path_len=plen, status=st,
                        stream=stream)

    def commit_only(i):
        p = pools[i % len(pools)]
        G.commit(p["S0"], p["U"], p["k"], p["g"], p["off"], p["par"], p["path"], p["plen"], max_nodes=mn,
                 S_out=p["S_out"], status=st, stream=stream)

    def replay(i):
        p = pools[i % len(pools)]
        G.commit_replay(p["S0"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"], p["path"], p["plen"],
                        max_nodes=mn, S_out=p["S_out"], status=st, stream=stream)

    t_path = _time_launches(path_only, n, stream)
    t_commit = _time_launches(commit_only, n, stream)
    cb_step = commit_bytes(wl, pools[0]["plen"].cpu().numpy())
    t_greedy = _time_launches(greedy, n, stream)
    t_fused = _time_launches(fused, n, stream)
    L = plen.cpu().numpy()
    cb = commit_bytes(wl, L)
    t_replay = _time_launches(replay, n, stream)
    Lr = pools[0]["plen"].cpu().numpy()
    # replay reads k and v rows and the two gates of each path node instead of U
    rb = int(commit_bytes(wl, Lr) - (wl.Hv * Lr * (4 * D + 4)).sum() + (wl.Hv * Lr * (2 * D + 8)).sum())
    # load-adaptive budget: half of the batch's nodes, no threshold
    prob = torch.from_numpy(W.acceptance_probs(wl)).to(dev)
    surv = torch.empty((wl.T,), dtype=torch.float32, device=dev)
    keep = torch.empty((wl.T,), dtype=torch.uint8, device=dev)
    kept = torch.empty((B,), dtype=torch.int32, device=dev)

    def budget(i):
        p = pools[i % len(pools)]
        G.budget_select(p["off"], p["par"], prob, wl.T // 2, 0.0, max_nodes=mn, survival=surv, keep=keep,
                        kept=kept, status=st, stream=stream)

    t_budget = _time_launches(budget, n, stream)
    # greedy acceptance, commit and the next tree's verify in one launch
    cst2 = torch.empty((B,), dtype=torch.int32, device=dev)
    tok = dict(draft_token=dt, target_token=tg, root_token=rt)

    def greedy_step(i):
        p = pools[i % len(pools)]
        prev = dict(U=p["U"], k=p["k"], g=p["g"], node_offset=p["off"], parent=p["par"], max_nodes=mn)
        G.commit_verify(p["S0"], prev, acc, p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"],
                        max_nodes=mn, S_out=p["S_out"], out=p["out2"], U=p["U2"], anc_mask=p["anc"], status=st,
                        commit_status=cst2, stream=stream, greedy=tok)

    t_gcv = _time_launches(greedy_step, n, stream)
    gcv_b = verify_bytes(wl) + cb - wl.B * wl.Hv * D * D * 4
    # the one-launch step in place (S_out = S0, as a serving loop keeps one state per slot):
    # requests that accepted nothing write no state.  Each pool's state drifts from step to
    # step (the same path is committed again); only the timing is used.
    ip = [dict(S=p["S0"].clone()) for p in pools[:2]]

    def inplace_step(i):
        p, s = pools[i % 2], ip[i % 2]
        prev = dict(U=p["U"], k=p["k"], g=p["g"], node_offset=p["off"], parent=p["par"], max_nodes=mn)
        G.commit_verify(s["S"], prev, p["acc"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"],
                        max_nodes=mn, S_out=s["S"], out=p["out2"], U=p["U2"], anc_mask=p["anc"], status=st,
                        commit_status=cst2, stream=stream)

    t_ip = _time_launches(inplace_step, n, stream)
    L0 = pools[0]["plen"].cpu().numpy()
    ip_b = int(verify_bytes(wl) + commit_bytes(wl, L0) - wl.B * wl.Hv * D * D * 4
               - (L0 == 0).sum() * wl.Hv * D * D * 4)   # no state write where nothing was accepted
    del ip
    return {"accepted_path_then_commit": {"accepted_path_avg_us": t_path, "commit_avg_us": t_commit,
                                          "commit_alg_GBps": cb_step / (t_commit * 1e-6) / 1e9,
                                          "commit_hbm_frac": cb_step / (t_commit * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "budget_select": {"avg_us": t_budget, "budget": wl.T // 2, "nodes": wl.T},
            "commit_replay": {"avg_us": t_replay, "alg_bytes": rb, "alg_GBps": rb / (t_replay * 1e-6) / 1e9,
                              "hbm_frac": rb / (t_replay * 1e-6) / 1e9 / HBM_PEAK_GBS,
                              "mean_accepted_len": float(Lr.mean())},
            "accept_greedy": {"avg_us": t_greedy, "mean_accepted_len": float(L.mean())},
            "commit_verify_in_place": {"avg_us": t_ip, "alg_bytes": ip_b, "nodes_per_s": wl.T / (t_ip * 1e-6),
                                       "alg_GBps": ip_b / (t_ip * 1e-6) / 1e9,
                                       "hbm_frac": ip_b / (t_ip * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                       "requests_without_state_write": int((L0 == 0).sum())},
            "accept_commit_verify": {"avg_us": t_gcv, "alg_bytes": gcv_b,
                                     "alg_GBps": gcv_b / (t_gcv * 1e-6) / 1e9,
                                     "hbm_frac": gcv_b / (t_gcv * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "accept_commit_fused": {"avg_us": t_fused, "alg_bytes": cb,
                                    "alg_GBps": cb / (t_fused * 1e-6) / 1e9,
                                    "hbm_frac": cb / (t_fused * 1e-6) / 1e9 / HBM_PEAK_GBS}}

def attention_bytes(wl):
    """Algorithmic HBM bytes of one tree-bias attention launch: every context
    key/value row once per kv head, the nodes' own keys/values, q, out, lse and
    the masks."""
    import numpy as np
    C = int(wl.ctx_offset[-1])
    return int(C * wl.Hkv * 2 * D * 2 + wl.T * wl.Hkv * 2 * D * 2 + wl.T * wl.Hq * (D * 2 + D * 4 + 4)
               + wl.T * 8 + 2 * (wl.B + 1) * 4)


def attention_row(args, stream):
    """Tree-bias attention of the hybrid's attention layers over the batch-256
    mixed trees with contexts of 1k-4k tokens (32 query / 8 kv heads)."""
    import numpy as np
    import torch
    import workloads as W
    from speculative_decoding_tree_amd import gdn_tree as G
    t0 = time.time()
    wl = W.make_attn_mixed_b256(0)
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    q, kc, vc, kn, vn = bf(wl.q), bf(wl.k_ctx), bf(wl.v_ctx), bf(wl.k_node), bf(wl.v_node)
    co, no, par = i32(wl.ctx_offset), i32(wl.node_offset), i32(wl.parent)
    print(f"[bench] tree attention inputs: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} T={wl.T} context rows={wl.C} "
          f"in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    mn, mc = wl.max_nodes, wl.max_ctx
    anc = torch.empty((wl.T,), dtype=torch.int64, device=dev)
    st = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    out = torch.empty((wl.T, wl.Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=dev)
    n = max(10, args.steps // 4)
    t_anc = _time_launches(lambda i: G.ancestry(no, par, max_nodes=mn, anc_mask=anc, status=st, stream=stream),
                           n, stream)
    res = {"workload": "mixed batch-256 trees, contexts U[1024, 4096], Hq=32, Hkv=8, d=128",
           "context_rows": wl.C, "nodes": wl.T, "ancestry_avg_us": t_anc}
    nbytes = attention_bytes(wl)
    for split in (None, 1024):
        ws_need = G.attention_workspace_bytes(G.make_attn_dims(wl.B, wl.Hq, wl.Hkv, wl.T, wl.C, mn, mc, split))
        ws = torch.empty((max(ws_need, 16),), dtype=torch.uint8, device=dev)

        def run(i, split=split, ws=ws):
            G.attention(q, kc, vc, co, kn, vn, no, anc, wl.scale, max_nodes=mn, max_ctx=mc, split=split,
                        out=out, lse=lse, workspace=ws, status=st, stream=stream)
        t = _time_launches(run, n, stream)
        key = "one_pass" if split is None else f"split_{split}"
        res[key] = {"avg_us": t, "alg_bytes": nbytes, "alg_GBps": nbytes / (t * 1e-6) / 1e9,
                    "hbm_frac": nbytes / (t * 1e-6) / 1e9 / HBM_PEAK_GBS}
        if split is None:
            res[key]["hbm_traffic_bytes"] = measured_traffic("mixed_b256", "gdn_tree_attention")
    assert (st.cpu().numpy() == 0).all()

    # batch one: the six-node root-branch tree over a 4096-token context, where one pass has
    # only Hkv workgroups of work and splitting the context spreads it over more
    w1 = W.make_attn([W.root_branch()], [4096], Hq=wl.Hq, Hkv=wl.Hkv, seed=3, name="attn_b1")
    q1, kc1, vc1, kn1, vn1 = bf(w1.q), bf(w1.k_ctx), bf(w1.v_ctx), bf(w1.k_node), bf(w1.v_node)
    co1, no1, par1 = i32(w1.ctx_offset), i32(w1.node_offset), i32(w1.parent)
    anc1 = torch.empty((w1.T,), dtype=torch.int64, device=dev)
    st1 = torch.empty((1,), dtype=torch.int32, device=dev)
    G.ancestry(no1, par1, max_nodes=w1.max_nodes, anc_mask=anc1, status=st1, stream=stream)
    out1 = torch.empty((w1.T, w1.Hq, D), dtype=torch.float32, device=dev)
    lse1 = torch.empty((w1.T, w1.Hq), dtype=torch.float32, device=dev)
    b1 = {"workload": "1 request, 6-node root-branch tree, 4096-token context, Hq=32, Hkv=8, d=128"}
    for split in (None, 1024, 256, 0):
        ws_need = G.attention_workspace_bytes(G.make_attn_dims(1, w1.Hq, w1.Hkv, w1.T, w1.C, w1.max_nodes, w1.C,
                                                                split))
        ws = torch.empty((max(ws_need, 16),), dtype=torch.uint8, device=dev)

        def run1(i, split=split, ws=ws):
            G.attention(q1, kc1, vc1, co1, kn1, vn1, no1, anc1, w1.scale, max_nodes=w1.max_nodes, max_ctx=w1.C,
                        split=split, out=out1, lse=lse1, workspace=ws, status=st1, stream=stream)
        key = "one_pass_us" if split is None else ("split_chosen_us" if split == 0 else f"split_{split}_us")
        b1[key] = _time_launches(run1, n, stream)
    assert (st1.cpu().numpy() == 0).all()
    res["batch_one"] = b1
    return res


def batch_one_row(args, stream):
    """Latency of one step at batch one, as verify + commit_node launches
    (eager and captured in a HIP graph) and as one commit_verify launch (eager
    and captured): the 6-node root-branch tree of one request, 32 value / 16
    key heads (the shape of the batch-one decode gate the pages report)."""
    import numpy as np
    import torch
    import workloads as W
    from speculative_decoding_tree_amd import gdn_tree as G
    wl = W.make_root_branch6(B=1)
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    S0, q, k, v, g, beta = f32(wl.S0), bf(wl.q), bf(wl.k), bf(wl.v), f32(wl.g), f32(wl.beta)
    off, par, acc = i32(wl.node_offset), i32(wl.parent), i32(wl.accept_node)
    mn = wl.max_nodes
    out = torch.empty((wl.T, wl.Hv, D), dtype=torch.float32, device=dev)
    U = torch.empty_like(out)
    anc = torch.empty((wl.T,), dtype=torch.int64, device=dev)
    st = torch.empty((1,), dtype=torch.int32, device=dev)
    path = torch.empty((1, mn), dtype=torch.int32, device=dev)
    plen = torch.empty((1,), dtype=torch.int32, device=dev)
    S1 = torch.empty_like(S0)

    def step(i):
        G.verify(S0, q, k, v, g, beta, off, par, max_nodes=mn, out=out, U=U, anc_mask=anc, status=st, stream=stream)
        G.commit_node(S0, U, k, g, off, par, acc, max_nodes=mn, S_out=S1, path=path, path_len=plen, status=st,
                      stream=stream)

    t = _time_launches(step, max(20, args.steps), stream)
    # the same step captured once in a HIP graph and replayed (no per-launch host cost)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(0)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.verify(S0, q, k, v, g, beta, off, par, max_nodes=mn, out=out, U=U, anc_mask=anc, status=st)
        G.commit_node(S0, U, k, g, off, par, acc, max_nodes=mn, S_out=S1, path=path, path_len=plen, status=st)
    t_graph = _time_launches(lambda i: graph.replay(), max(20, args.steps), stream)
    # the fused step: the previous tree's commit and this tree's verify in one launch
    out2, U2 = torch.empty_like(out), torch.empty_like(U)
    prev = dict(U=U, k=k, g=g, node_offset=off, parent=par, max_nodes=mn)

    def fstep(i):
        G.commit_verify(S0, prev, acc, q, k, v, g, beta, off, par, max_nodes=mn, S_out=S1, out=out2, U=U2,
                        anc_mask=anc, status=st, commit_status=plen, stream=stream)

    t_fused = _time_launches(fstep, max(20, args.steps), stream)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fstep(0)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    fgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(fgraph):
        G.commit_verify(S0, prev, acc, q, k, v, g, beta, off, par, max_nodes=mn, S_out=S1, out=out2, U=U2,
                        anc_mask=anc, status=st, commit_status=plen)
    t_fgraph = _time_launches(lambda i: fgraph.replay(), max(20, args.steps), stream)
    return {"workload": "1 request, 6-node root-branch tree, Hv=32, Hk=16, d=128", "step_us": t,
            "graph_step_us": t_graph, "commit_verify_step_us": t_fused, "commit_verify_graph_step_us": t_fgraph}


def config_rows(args, stream):
    """The other workloads the pages' shapes give (depth-3 chains at batch 64, the
    6-node root-branch tree at batch 16 and 1, random 32-node trees at batch 256):
    the one-launch step (gdn_tree_commit_verify, the batch playing both trees, out
    of place) and the two-launch step (gdn_tree_verify + gdn_tree_commit_node),
    each with nodes/s, commits/s and its fraction of the HBM peak.  Three copies of
    every buffer rotate, as in the headline loop.  Each step is timed launched from
    Python and replayed from a HIP graph (graph_*: no per-launch host cost, which
    decides the small batches' times)."""
    import numpy as np
    import torch
    import workloads as W
    from speculative_decoding_tree_amd import gdn_tree as G
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    rows = {}
    makers = (("chain3_b64", W.make_chain3_b64), ("rootbranch6_b16", lambda: W.make_root_branch6(B=16)),
              ("rootbranch6_b1", lambda: W.make_root_branch6(B=1)), ("random32_b256", W.make_random32_b256))
    n = max(20, args.steps // 2)
    for name, make in makers:
        wl = make()
        mn = wl.max_nodes
        pools = []
        for _ in range(max(1, args.pools)):
            p = dict(S0=torch.from_numpy(wl.S0).to(dev), q=bf(wl.q), k=bf(wl.k), v=bf(wl.v),
                     g=torch.from_numpy(wl.g).to(dev), beta=torch.from_numpy(wl.beta).to(dev),
                     off=torch.from_numpy(wl.node_offset).to(dev), par=torch.from_numpy(wl.parent).to(dev),
                     acc=torch.from_numpy(wl.accept_node).to(dev))
            p["S_out"] = torch.empty_like(p["S0"])
            for key in ("out", "U", "out2", "U2"):
                p[key] = torch.empty((wl.T, wl.Hv, D), dtype=torch.float32, device=dev)
            p["anc"] = torch.empty((wl.T,), dtype=torch.int64, device=dev)
            for key in ("st", "cst", "plen"):
                p[key] = torch.empty((wl.B,), dtype=torch.int32, device=dev)
            p["path"] = torch.empty((wl.B, mn), dtype=torch.int32, device=dev)
            pools.append(p)

        def two(i):
            p = pools[i % len(pools)]
            G.verify(p["S0"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"], max_nodes=mn,
                     out=p["out"], U=p["U"], anc_mask=p["anc"], status=p["st"], stream=stream)
            G.commit_node(p["S0"], p["U"], p["k"], p["g"], p["off"], p["par"], p["acc"], max_nodes=mn,
                          S_out=p["S_out"], path=p["path"], path_len=p["plen"], status=p["cst"], stream=stream)

        def one(i):
            p = pools[i % len(pools)]
            prev = dict(U=p["U"], k=p["k"], g=p["g"], node_offset=p["off"], parent=p["par"], max_nodes=mn)
            G.commit_verify(p["S0"], prev, p["acc"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"],
                            max_nodes=mn, S_out=p["S_out"], out=p["out2"], U=p["U2"], anc_mask=p["anc"],
                            status=p["st"], commit_status=p["cst"], path=p["path"], path_len=p["plen"],
                            stream=stream)

        t_two = _time_launches(two, n, stream)      # also leaves every pool's U for the one-launch step
        t_one = _time_launches(one, n, stream)

        # the same steps replayed from a HIP graph (one step per pool per replay), which takes
        # the Python binding's per-launch cost out of the timed interval
        def graph_of(fn):
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for i in range(len(pools)):
                    fn(i, None)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(len(pools)):
                    fn(i, None)
            return gr

        def two_s(i, s):
            p = pools[i % len(pools)]
            G.verify(p["S0"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"], max_nodes=mn,
                     out=p["out"], U=p["U"], anc_mask=p["anc"], status=p["st"], stream=s)
            G.commit_node(p["S0"], p["U"], p["k"], p["g"], p["off"], p["par"], p["acc"], max_nodes=mn,
                          S_out=p["S_out"], path=p["path"], path_len=p["plen"], status=p["cst"], stream=s)

        def one_s(i, s):
            p = pools[i % len(pools)]
            prev = dict(U=p["U"], k=p["k"], g=p["g"], node_offset=p["off"], parent=p["par"], max_nodes=mn)
            G.commit_verify(p["S0"], prev, p["acc"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"],
                            max_nodes=mn, S_out=p["S_out"], out=p["out2"], U=p["U2"], anc_mask=p["anc"],
                            status=p["st"], commit_status=p["cst"], path=p["path"], path_len=p["plen"], stream=s)
        g_two, g_one = graph_of(two_s), graph_of(one_s)
        t_two_g = _time_launches(lambda i: g_two.replay(), n, stream) / len(pools)
        t_one_g = _time_launches(lambda i: g_one.replay(), n, stream) / len(pools)
        del g_two, g_one
        st = np.concatenate([p["st"].cpu().numpy() for p in pools] + [p["cst"].cpu().numpy() for p in pools])
        if not (st == 0).all():
            raise RuntimeError(f"{name}: device status nonzero")
        L = pools[0]["plen"].cpu().numpy()
        vb, cb = verify_bytes(wl), commit_bytes(wl, L)
        fb = vb + cb - wl.B * wl.Hv * D * D * 4
        rows[name] = {
            "B": wl.B, "Hv": wl.Hv, "Hk": wl.Hk, "T": wl.T, "max_nodes": mn, "mean_accepted_len": float(L.mean()),
            "one_launch": {"avg_us": t_one, "nodes_per_s": wl.T / (t_one * 1e-6), "commits_per_s": wl.B / (t_one * 1e-6),
                           "alg_bytes": fb, "alg_GBps": fb / (t_one * 1e-6) / 1e9,
                           "hbm_frac": fb / (t_one * 1e-6) / 1e9 / HBM_PEAK_GBS,
                           "graph_avg_us": t_one_g, "graph_nodes_per_s": wl.T / (t_one_g * 1e-6),
                           "graph_hbm_frac": fb / (t_one_g * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "two_launch": {"avg_us": t_two, "nodes_per_s": wl.T / (t_two * 1e-6), "commits_per_s": wl.B / (t_two * 1e-6),
                           "alg_bytes": vb + cb, "alg_GBps": (vb + cb) / (t_two * 1e-6) / 1e9,
                           "hbm_frac": (vb + cb) / (t_two * 1e-6) / 1e9 / HBM_PEAK_GBS,
                           "graph_avg_us": t_two_g, "graph_nodes_per_s": wl.T / (t_two_g * 1e-6),
                           "graph_hbm_frac": (vb + cb) / (t_two_g * 1e-6) / 1e9 / HBM_PEAK_GBS}}
        del pools
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed_b256", choices=["mixed_b256", "random32_b256"])
    ap.add_argument("--pools", type=int, default=3, help="rotated copies of every buffer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-storeall", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=256, help="requests in the oracle sample")
    ap.add_argument("--no-next", action="store_true", help="skip the next-row measurements")
    ap.add_argument("--no-attention", action="store_true", help="skip the tree-bias attention measurement")
    ap.add_argument("--no-batch-one", action="store_true", help="skip the batch-one latency measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' rows")
    ap.add_argument("--batch-one-only", action="store_true",
                    help="only the batch-one latency rows (one JSON line), e.g. under a kernel trace")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the verify/commit path has no cross-GPU step and this "
              "build runs on a single MI355X; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from speculative_decoding_tree_amd import gdn_tree as G

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X visible to torch", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    if args.batch_one_only:
        print(json.dumps({"batch_one": batch_one_row(args, torch.cuda.current_stream())}), flush=True)
        return

    t0 = time.time()
    wl = W.make_mixed_b256() if args.workload == "mixed_b256" else W.make_random32_b256()
    log(f"[bench] generated {wl.name}: B={wl.B} Hv={wl.Hv} Hk={wl.Hk} T={wl.T} "
        f"max_nodes={wl.max_nodes} in {time.time() - t0:.1f}s")
    mn = wl.max_nodes
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def make_pool():
        p = dict(S0=torch.from_numpy(wl.S0).to(dev), q=bf(wl.q), k=bf(wl.k), v=bf(wl.v),
                 g=torch.from_numpy(wl.g).to(dev), beta=torch.from_numpy(wl.beta).to(dev),
                 off=torch.from_numpy(wl.node_offset).to(dev), par=torch.from_numpy(wl.parent).to(dev),
                 acc=torch.from_numpy(wl.accept_node).to(dev))
        p["S_out"] = torch.empty_like(p["S0"])
        p["out"] = torch.empty((wl.T, wl.Hv, D), dtype=torch.float32, device=dev)
        p["U"] = torch.empty_like(p["out"])
        p["anc"] = torch.empty((wl.T,), dtype=torch.int64, device=dev)
        p["status"] = torch.empty((wl.B,), dtype=torch.int32, device=dev)
        p["path"] = torch.empty((wl.B, mn), dtype=torch.int32, device=dev)
        p["plen"] = torch.empty((wl.B,), dtype=torch.int32, device=dev)
        p["pst"] = torch.empty((wl.B,), dtype=torch.int32, device=dev)
        p["cst"] = torch.empty((wl.B,), dtype=torch.int32, device=dev)
        return p

    pools = [make_pool() for _ in range(max(1, args.pools))]
    stream = torch.cuda.current_stream()

    def step(p, ev=None):
        if ev is not None:
            ev[0].record(stream)
        G.verify(p["S0"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"], max_nodes=mn,
                 out=p["out"], U=p["U"], anc_mask=p["anc"], status=p["status"], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        G.commit_node(p["S0"], p["U"], p["k"], p["g"], p["off"], p["par"], p["acc"], max_nodes=mn,
                      S_out=p["S_out"], path=p["path"], path_len=p["plen"], status=p["cst"], stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(pools[i % len(pools)])
    torch.cuda.synchronize()
    st = pools[0]["status"].cpu().numpy()
    if not (np.all(st == 0) and np.all(pools[0]["cst"].cpu().numpy() == 0)):
        raise RuntimeError(f"device status nonzero: {st}")
    path_len = pools[0]["plen"].cpu().numpy()

    # timed region: whole steps only
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(pools[i % len(pools)])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps

    # per-kernel durations: events around each launch (separate pass, same steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(pools[i % len(pools)], evs[i])
    torch.cuda.synchronize()
    t_ver = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3     # us
    t_com = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3

    vb, cb = verify_bytes(wl), commit_bytes(wl, path_len)
    vf = verify_flops(wl)

    def kstats(t, nbytes, flops=None):
        d = {"avg_us": float(t.mean()), "p10_us": float(np.percentile(t, 10)),
             "p50_us": float(np.percentile(t, 50)), "p90_us": float(np.percentile(t, 90)),
             "alg_bytes": nbytes, "alg_GBps": nbytes / (t.mean() * 1e-6) / 1e9,
             "hbm_frac": nbytes / (t.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS}
        if flops:
            d["alg_flops"] = flops
            d["TFLOPs"] = flops / (t.mean() * 1e-6) / 1e12
        return d

    kernels = {"gdn_tree_verify": kstats(t_ver, vb, vf), "gdn_tree_commit_node": kstats(t_com, cb)}
    dom = max(("gdn_tree_verify", "gdn_tree_commit_node"), key=lambda k: kernels[k]["avg_us"])
    ach = kernels[dom]["alg_GBps"]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name, dom),
                "alg_bytes_per_launch": kernels[dom]["alg_bytes"]}
    for kname in ("gdn_tree_verify", "gdn_tree_commit_node"):
        kernels[kname]["hbm_traffic_bytes"] = measured_traffic(wl.name, kname)

    # The previous tree's commit fused with the next tree's verify: one launch per
    # step that reads each state once (the same batch plays both trees; its U from
    # the separate steps above is the previous tree's pseudo-values).
    for p in pools:
        p["out2"] = torch.empty_like(p["out"])
        p["U2"] = torch.empty_like(p["U"])

    def fstep(p):
        prev = dict(U=p["U"], k=p["k"], g=p["g"], node_offset=p["off"], parent=p["par"], max_nodes=mn)
        G.commit_verify(p["S0"], prev, p["acc"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"],
                        max_nodes=mn, S_out=p["S_out"], out=p["out2"], U=p["U2"], anc_mask=p["anc"],
                        status=p["status"], commit_status=p["cst"], path=p["path"], path_len=p["plen"],
                        stream=stream)

    for i in range(args.warmup):
        fstep(pools[i % len(pools)])
    torch.cuda.synchronize()
    if not (np.all(pools[0]["status"].cpu().numpy() == 0) and np.all(pools[0]["cst"].cpu().numpy() == 0)):
        raise RuntimeError("device status nonzero in commit_verify")
    # timed region (headline): whole fused steps only.  One event on the launch
    # stream at every step boundary: the first and last bracket the region, and
    # consecutive pairs give each launch's duration (gaps included).
    fev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    fev[0].record(stream)
    for i in range(args.steps):
        fstep(pools[i % len(pools)])
        fev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_fused = fev[0].elapsed_time(fev[-1]) / args.steps
    t_fus = np.array([fev[i].elapsed_time(fev[i + 1]) for i in range(args.steps)]) * 1e3
    fb = vb + cb - wl.B * wl.Hv * D * D * 4   # the committed state is not read back
    fkern = {"gdn_tree_commit_verify": kstats(t_fus, fb, vf)}
    fkern["gdn_tree_commit_verify"]["hbm_traffic_bytes"] = measured_traffic(wl.name, "gdn_tree_commit_verify")
    fach = fkern["gdn_tree_commit_verify"]["alg_GBps"]
    froof = {"bound": "hbm", "kernel": "gdn_tree_commit_verify", "achieved": fach, "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": fach / HBM_PEAK_GBS,
             "traffic": measured_traffic(wl.name, "gdn_tree_commit_verify"), "alg_bytes_per_launch": fb}
    separate = {"ms_per_step": ms_step, "nodes_per_s": wl.T / (ms_step * 1e-3),
                "commits_per_s": wl.B / (ms_step * 1e-3),
                "hbm_frac_step": (vb + cb) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "roofline": roofline, "kernels": kernels}

    nodes_per_s = wl.T / (ms_fused * 1e-3)
    result = {
        "metric": METRIC, "value": nodes_per_s, "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_fused, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 hi/lo MFMA, fp32 accumulate", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Hv": wl.Hv, "Hk": wl.Hk, "d_k": D, "d_v": D, "T": wl.T,
                   "max_nodes": mn, "trees": ("64 each of chain-3, root-branch-6, random-16, random-64"
                                              if args.workload == "mixed_b256" else "random-32, depth <= 6"),
                   "inputs": "q/k/v bf16, S0/g/beta fp32, seed 0", "parallelism": "single-gpu"},
        "step": "gdn_tree_commit_verify: the previous tree's commit and this tree's verify, one launch",
        "commits_per_s": wl.B / (ms_fused * 1e-3),
        "node_heads_per_s": wl.T * wl.Hv / (ms_fused * 1e-3),
        "hbm_frac_step": fb / (ms_fused * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": froof, "kernels": fkern,
        "separate_step": separate,
    }

    if not args.no_storeall:
        p = pools[0]
        node_state = torch.empty((wl.T, wl.Hv, D, D), dtype=torch.float32, device=dev)
        sa_out = torch.empty_like(p["out"])
        sa_S = torch.empty_like(p["S0"])
        sa_st = torch.empty((wl.B,), dtype=torch.int32, device=dev)

        def sa_step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            G.verify_storeall(p["S0"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["off"], p["par"],
                              max_nodes=mn, out=sa_out, node_state=node_state, status=sa_st, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            G.commit_storeall(p["S0"], node_state, p["off"], p["par"], p["acc"], max_nodes=mn, S_out=sa_S,
                              status=sa_st, stream=stream)
            if ev is not None:
                ev[2].record(stream)

        for _ in range(3):
            sa_step()
        n_sa = max(5, args.steps // 5)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_sa)]
        torch.cuda.synchronize()
        for i in range(n_sa):
            sa_step(sev[i])
        torch.cuda.synchronize()
        sv = np.array([e[0].elapsed_time(e[1]) for e in sev]) * 1e3
        sc = np.array([e[1].elapsed_time(e[2]) for e in sev]) * 1e3
        dims = G.make_dims(wl.B, wl.Hv, wl.Hk, wl.T, mn, wl.B)
        result["storeall"] = {
            "verify_avg_us": float(sv.mean()), "commit_avg_us": float(sc.mean()),
            "ms_per_step": float((sv.mean() + sc.mean()) * 1e-3),
            "speculative_state_bytes": G.state_bytes(dims, True),
            "treewy_speculative_state_bytes": G.state_bytes(dims, False),
            "node_state_write_GBps": wl.T * wl.Hv * D * D * 4 / (sv.mean() * 1e-6) / 1e9,
            "treewy_ms_per_step": ms_step,
            "treewy_commit_verify_ms_per_step": ms_fused,
        }
        del node_state
        torch.cuda.empty_cache()

    if not args.no_next:
        result["next_rows"] = next_rows(args, wl, pools, mn, stream)
        if not args.no_attention:
            result["next_rows"]["tree_attention"] = attention_row(args, stream)
        if not args.no_batch_one:
            result["next_rows"]["batch_one"] = batch_one_row(args, stream)

    if not args.no_configs:
        result["configs"] = config_rows(args, stream)

    # the same GPU's runtime device-to-device copy (1 GiB read + 1 GiB written), for
    # context beside a kernel that reads each state once and writes it once
    ca = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cb = torch.empty_like(ca)
    t_copy = _time_launches(lambda i: cb.copy_(ca), 10, stream)
    copy_gbps = 2 * ca.numel() * 4 / (t_copy * 1e-6) / 1e9
    result["device_copy"] = {"what": "runtime device-to-device copy (hipMemcpyAsync), 1 GiB each way",
                             "GBps": copy_gbps, "frac": copy_gbps / HBM_PEAK_GBS, "bytes": 2 * ca.numel() * 4,
                             "avg_us": t_copy}
    del ca, cb
    torch.cuda.empty_cache()

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 2 * a.numel() * 4

    if not args.no_cpu_baseline:
        log(f"[bench] oracle sample: {args.cpu_sample} requests on host cores")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
