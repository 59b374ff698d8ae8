"""HIP-graph capture of the entry points.

The library only enqueues kernels (no allocation, synchronisation or memset),
so a decode step can be captured once and replayed.  Each test captures a step,
then replays it several times with unrelated eager work, output poisoning and
synchronisations in between; every replay must reproduce the eager results bit
for bit (same kernels, same inputs).
"""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import host, upload

import speculative_decoding_tree_amd.gdn_tree as G

pytestmark = pytest.mark.gpu


def _capture(step):
    """Warm up on a side stream (as torch's capture expects), then capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    return graph


def _replays_match(graph, outputs, poison, ref, reps=4):
    junk = torch.randn(1 << 20, device=outputs[0].device)
    for _ in range(reps):
        poison()
        junk.mul_(1.0001)                     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, ref):
            assert np.array_equal(host(got), want)


def test_verify_path_commit_step_replays_bit_exact():
    wl = W.make_root_branch6(16)
    u = upload(wl)
    mn, d = wl.max_nodes, u["S0"].device
    out = torch.empty((wl.T, wl.Hv, 128), dtype=torch.float32, device=d)
    U = torch.empty_like(out)
    anc = torch.empty((wl.T,), dtype=torch.int64, device=d)
    st = torch.empty((wl.B,), dtype=torch.int32, device=d)
    path = torch.empty((wl.B, mn), dtype=torch.int32, device=d)
    plen = torch.empty((wl.B,), dtype=torch.int32, device=d)
    S1 = torch.empty_like(u["S0"])

    def step():
        G.verify(u["S0"], u["q"], u["k"], u["v"], u["g"], u["beta"], u["node_offset"], u["parent"],
                 max_nodes=mn, out=out, U=U, anc_mask=anc, status=st)
        G.accepted_path(u["node_offset"], u["parent"], u["accept_node"], max_nodes=mn, path=path,
                        path_len=plen, status=st)
        G.commit(u["S0"], U, u["k"], u["g"], u["node_offset"], u["parent"], path, plen, max_nodes=mn,
                 S_out=S1, status=st)

    step()
    torch.cuda.synchronize()
    outputs = (out, U, anc, path, plen, S1, st)
    ref = [host(x).copy() for x in outputs]
    assert (ref[-1] == 0).all()

    def poison():
        for x in (out, U, S1):
            x.fill_(float("nan"))
        for x in (path, plen, st):
            x.fill_(-7)
        anc.fill_(0)

    _replays_match(_capture(step), outputs, poison, ref)


def test_commit_verify_step_replays_bit_exact():
    """The one-launch step (previous tree's commit, next tree's verify) captured and replayed."""
    P, C = W.make_root_branch6(16), W.make_root_branch6(16, seed=1)
    uP, uC = upload(P), upload(C)
    mn, d = P.max_nodes, uP["S0"].device
    _, U_P, _, _ = G.verify(uP["S0"], uP["q"], uP["k"], uP["v"], uP["g"], uP["beta"], uP["node_offset"],
                            uP["parent"], max_nodes=mn)
    prev = dict(U=U_P, k=uP["k"], g=uP["g"], node_offset=uP["node_offset"], parent=uP["parent"], max_nodes=mn)
    out = torch.empty((C.T, C.Hv, 128), dtype=torch.float32, device=d)
    U = torch.empty_like(out)
    anc = torch.empty((C.T,), dtype=torch.int64, device=d)
    st = torch.empty((C.B,), dtype=torch.int32, device=d)
    cst = torch.empty((C.B,), dtype=torch.int32, device=d)
    S1 = torch.empty_like(uP["S0"])

    def step():
        G.commit_verify(uP["S0"], prev, uP["accept_node"], uC["q"], uC["k"], uC["v"], uC["g"], uC["beta"],
                        uC["node_offset"], uC["parent"], max_nodes=mn, S_out=S1, out=out, U=U, anc_mask=anc,
                        status=st, commit_status=cst)

    step()
    torch.cuda.synchronize()
    outputs = (S1, out, U, anc, st, cst)
    ref = [host(x).copy() for x in outputs]
    assert (ref[-1] == 0).all() and (ref[-2] == 0).all()

    def poison():
        for x in (out, U, S1):
            x.fill_(float("nan"))
        for x in (st, cst):
            x.fill_(-7)
        anc.fill_(0)

    _replays_match(_capture(step), outputs, poison, ref)


@pytest.mark.parametrize("split", [None, 64])
def test_attention_replays_bit_exact(split):
    # the scheduled launch is a counter-reset kernel plus the attention kernel
    wl = W.make_attn_small(7)
    d = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d).view(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(d)
    q, kc, vc, kn, vn = bf(wl.q), bf(wl.k_ctx), bf(wl.v_ctx), bf(wl.k_node), bf(wl.v_node)
    co, no, par = i32(wl.ctx_offset), i32(wl.node_offset), i32(wl.parent)
    mn = max(1, wl.max_nodes)
    dims = G.make_attn_dims(wl.B, wl.Hq, wl.Hkv, wl.T, wl.C, mn, wl.max_ctx, split)
    ws = torch.empty((G.attention_workspace_bytes(dims),), dtype=torch.uint8, device=d)
    anc = torch.empty((wl.T,), dtype=torch.int64, device=d)
    out = torch.empty((wl.T, wl.Hq, 128), dtype=torch.float32, device=d)
    lse = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=d)
    st = torch.empty((wl.B,), dtype=torch.int32, device=d)

    def step():
        G.ancestry(no, par, max_nodes=mn, anc_mask=anc, status=st)
        G.attention(q, kc, vc, co, kn, vn, no, anc, wl.scale, max_nodes=mn, max_ctx=wl.max_ctx, split=split,
                    out=out, lse=lse, workspace=ws, status=st)

    step()
    torch.cuda.synchronize()
    outputs = (anc, out, lse, st)
    ref = [host(x).copy() for x in outputs]
    assert (ref[-1] == 0).all()

    def poison():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        anc.fill_(0)
        st.fill_(-7)
        ws.fill_(0xAB)                        # the counters must be re-zeroed by the graph itself

    _replays_match(_capture(step), outputs, poison, ref)
