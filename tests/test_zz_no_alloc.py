"""GPU check of gdn_tree_attention_static, the allocation-free form of
gdn_tree_attention: through the C ABI, on two calls in a row (the second with a
smaller batch, so it runs over what the first left in the static scratch), in
one pass and with a split context, its outputs, log-sum-exps and statuses equal
those of gdn_tree_attention with a caller-owned workspace, bit for bit, and
meet the oracle's bar."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import tree_attention as A

import speculative_decoding_tree_amd.gdn_tree as G

pytestmark = pytest.mark.gpu

ATTN_TOL = 1e-4


def _upload(wl):
    d = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d).view(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(d)
    u = dict(q=bf(wl.q), k_ctx=bf(wl.k_ctx), v_ctx=bf(wl.v_ctx), k_node=bf(wl.k_node), v_node=bf(wl.v_node),
             ctx_offset=i32(wl.ctx_offset), node_offset=i32(wl.node_offset), parent=i32(wl.parent))
    u["anc"], _ = G.ancestry(u["node_offset"], u["parent"], max_nodes=max(1, wl.max_nodes))
    return u


def _both(wl, u, split):
    mn, mc = max(1, wl.max_nodes), wl.max_ctx
    args = (u["q"], u["k_ctx"], u["v_ctx"], u["ctx_offset"], u["k_node"], u["v_node"], u["node_offset"], u["anc"],
            wl.scale)
    dims = G.make_attn_dims(wl.B, wl.Hq, wl.Hkv, wl.T, wl.C, mn, mc, split)
    assert G.attention_workspace_bytes(dims) <= G.STATIC_SCRATCH_BYTES
    out_s = torch.full((wl.T, wl.Hq, 128), 7.0, device="cuda")
    lse_s = torch.full((wl.T, wl.Hq), 7.0, device="cuda")
    st_s = torch.full((wl.B,), 99, dtype=torch.int32, device="cuda")
    G.attention_static(*args, max_nodes=mn, max_ctx=mc, split=split, out=out_s, lse=lse_s, status=st_s)
    out_w, lse_w, st_w = G.attention(*args, max_nodes=mn, max_ctx=mc, split=split)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (out_s, lse_s, st_s, out_w, lse_w, st_w)]


def _smaller(wl, reqs):
    parents = [wl.parent[wl.node_offset[b]:wl.node_offset[b + 1]] for b in reqs]
    ctx = [int(wl.ctx_offset[b + 1] - wl.ctx_offset[b]) // 2 for b in reqs]
    return W.make_attn(parents, ctx, Hq=wl.Hq, Hkv=wl.Hkv, seed=77, name="attn_smaller")


@pytest.mark.parametrize("split", [None, 64, 0])
def test_attention_static_equals_workspace_entry_point(split):
    big = W.make_attn_small(4)
    small = _smaller(big, [5, 1, 2])
    for wl in (big, small):   # two calls in a row, the second smaller
        out_s, lse_s, st_s, out_w, lse_w, st_w = _both(wl, _upload(wl), split)
        assert np.array_equal(st_s, st_w) and (st_s == 0).all()
        rows = np.arange(wl.T)
        assert np.array_equal(out_s[rows].view(np.uint32), out_w[rows].view(np.uint32))
        assert np.array_equal(lse_s[rows].view(np.uint32), lse_w[rows].view(np.uint32))
        f = lambda x: W.bf16_bits_to_f32(x).astype(np.float64)
        ref_out, ref_lse, _ = A.tree_attention_batch(f(wl.q), f(wl.k_ctx), f(wl.v_ctx), wl.ctx_offset,
                                                     f(wl.k_node), f(wl.v_node), wl.node_offset, wl.parent,
                                                     wl.Hq, wl.Hkv, wl.scale, max_nodes=max(1, wl.max_nodes),
                                                     max_ctx=wl.max_ctx)
        err = np.abs(out_s - ref_out).max(axis=-1) / np.abs(ref_out).max(axis=-1)
        assert err.max() <= ATTN_TOL and np.abs(lse_s - ref_lse).max() <= ATTN_TOL


def test_attention_static_refuses_a_split_beyond_the_scratch():
    wl = W.make_attn_small(4)
    u = _upload(wl)
    with pytest.raises(G.GdnTreeError) as e:
        # 1-key parts: 8 requests x 2 kv heads x 200 parts x 4 row groups records exceed 64 MiB
        G.attention_static(u["q"], u["k_ctx"], u["v_ctx"], u["ctx_offset"], u["k_node"], u["v_node"],
                           u["node_offset"], u["anc"], wl.scale, max_nodes=wl.max_nodes, max_ctx=wl.max_ctx,
                           split=1)
    assert e.value.code == -10
