"""GPU parity of the tree-bias attention path through the C ABI against the fp64 oracle.

Bar: ancestry masks and statuses bit-exact; out row-normwise relative error
<= ATTN_TOL and |lse - lse_ref| <= ATTN_TOL.  The tolerance follows from the
arithmetic: q.k products of bf16 inputs are exact in fp32, softmax weights
enter the value product as bf16 hi + lo (relative error ~2^-17 = 7.6e-6 per
weight, random in sign), and what remains is fp32 accumulation over at most
max_ctx + 64 keys (~sqrt(4k) * 2^-24 = 4e-6 relative to sum |p v|).  1e-4
leaves a margin of ~20x over the errors these inputs show (~5e-6).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import gdn_oracle as O
from oracle import tree_attention as A
from helpers import anc_u64, host, rowwise_rel_err

import speculative_decoding_tree_amd.gdn_tree as G

pytestmark = pytest.mark.gpu

ATTN_TOL = 1e-4
# regression guard inside the bar: the errors these inputs show are ~5e-6 (out) and ~1.4e-6 (lse)
ATTN_ENVELOPE = 3e-5


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X visible to torch"
    return torch.device("cuda:0")


def upload_attn(wl):
    d = _dev()
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d).view(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(d)
    return dict(q=bf(wl.q), k_ctx=bf(wl.k_ctx), v_ctx=bf(wl.v_ctx), k_node=bf(wl.k_node), v_node=bf(wl.v_node),
                ctx_offset=i32(wl.ctx_offset), node_offset=i32(wl.node_offset), parent=i32(wl.parent))


def run_attn(wl, split=None, max_nodes=None, max_ctx=None, anc=None):
    d = upload_attn(wl)
    mn = max_nodes or max(1, wl.max_nodes)
    mc = wl.max_ctx if max_ctx is None else max_ctx
    if anc is None:
        anc, ast = G.ancestry(d["node_offset"], d["parent"], max_nodes=mn)
    out, lse, st = G.attention(d["q"], d["k_ctx"], d["v_ctx"], d["ctx_offset"], d["k_node"], d["v_node"],
                               d["node_offset"], anc, wl.scale, max_nodes=mn, max_ctx=mc, split=split)
    torch.cuda.synchronize()
    return host(out), host(lse), host(st), d


def oracle_attn(wl, requests=None, max_nodes=None, max_ctx=None):
    f = lambda x: W.bf16_bits_to_f32(x).astype(np.float64)
    return A.tree_attention_batch(f(wl.q), f(wl.k_ctx), f(wl.v_ctx), wl.ctx_offset, f(wl.k_node), f(wl.v_node),
                                  wl.node_offset, wl.parent, wl.Hq, wl.Hkv, wl.scale,
                                  max_nodes=max_nodes or max(1, wl.max_nodes),
                                  max_ctx=wl.max_ctx if max_ctx is None else max_ctx, requests=requests)


def rows_of(wl, reqs):
    return np.concatenate([np.arange(wl.node_offset[b], wl.node_offset[b + 1]) for b in reqs] +
                          [np.zeros(0, int)]).astype(int)


def compare(wl, out, lse, ref_out, ref_lse, reqs):
    rows = rows_of(wl, reqs)
    e = rowwise_rel_err(out[rows], ref_out[rows])
    el = float(np.abs(lse[rows] - ref_lse[rows]).max()) if rows.size else 0.0
    print(f"{wl.name}: out row-normwise rel err {e:.2e}, lse abs err {el:.2e}")
    assert e <= ATTN_TOL and e <= ATTN_ENVELOPE
    assert el <= ATTN_TOL and el <= ATTN_ENVELOPE


# ---- ancestry ----------------------------------------------------------------

@pytest.mark.parametrize("name", ["rootbranch6_b16", "mixed_b256"])
def test_ancestry_bit_exact(name):
    wl = W.make_mixed_b256() if name == "mixed_b256" else W.make_root_branch6(16)
    d = _dev()
    no = torch.from_numpy(wl.node_offset).to(d)
    par = torch.from_numpy(wl.parent).to(d)
    anc, st = G.ancestry(no, par, max_nodes=wl.max_nodes)
    ref = np.concatenate([np.array(O.ancestry(wl.parents_of(b)), dtype=np.uint64) for b in range(wl.B)])
    assert np.array_equal(anc_u64(anc), ref)
    assert (host(st) == 0).all()


def test_ancestry_matches_verify_masks():
    wl = W.make_custom([W.random_tree(np.random.default_rng(4), 40) for _ in range(6)], [0] * 6, Hv=4, Hk=2)
    d = _dev()
    from helpers import upload
    u = upload(wl)
    _, _, anc_v, _ = G.verify(u["S0"], u["q"], u["k"], u["v"], u["g"], u["beta"], u["node_offset"], u["parent"],
                              max_nodes=wl.max_nodes)
    anc_a, _ = G.ancestry(u["node_offset"], u["parent"], max_nodes=wl.max_nodes)
    assert np.array_equal(anc_u64(anc_v), anc_u64(anc_a))


def test_ancestry_statuses():
    d = _dev()
    # request 0 ok (chain), 1 bad parent (local parent[1] = 1), 2 too many (65 roots), 3 ends beyond T
    no = torch.tensor([0, 3, 6, 71, 72], dtype=torch.int32, device=d)
    par_h = np.array([-1, 0, 1, -1, 1, 1] + [-1] * 65, np.int32)
    par = torch.from_numpy(par_h).to(d)
    anc = torch.full((71,), -7, dtype=torch.int64, device=d)
    anc, st = G.ancestry(no, par, max_nodes=64, anc_mask=anc)
    st = host(st)
    assert list(st) == [O.STATUS_OK, O.STATUS_BAD_PARENT, O.STATUS_TOO_MANY_NODES, O.STATUS_BAD_OFFSETS]
    a = anc_u64(anc)
    assert list(a[:3]) == [1, 3, 7]
    assert (a[3:] == 0).all()


# ---- attention -----------------------------------------------------------------

@pytest.mark.parametrize("split", [None, 64, 100, 1])
def test_attention_small_full(split):
    wl = W.make_attn_small(0)
    out, lse, st, _ = run_attn(wl, split=split)
    ref_out, ref_lse, ref_st = oracle_attn(wl)
    assert np.array_equal(st, ref_st)
    compare(wl, out, lse, ref_out, ref_lse, range(wl.B))


def test_attention_split_agrees_with_one_pass():
    wl = W.make_attn_small(3)
    o1, l1, _, _ = run_attn(wl)
    o2, l2, _, _ = run_attn(wl, split=65)
    rows = rows_of(wl, range(wl.B))
    assert rowwise_rel_err(o2[rows], o1[rows]) <= ATTN_TOL
    assert np.abs(l2[rows] - l1[rows]).max() <= ATTN_TOL


def test_attention_no_context_at_all():
    parents = [W.chain(4), W.root_branch(), np.array([-1], np.int32)]
    wl = W.make_attn(parents, [0, 0, 0], Hq=4, Hkv=1, seed=9, name="attn_noctx")
    out, lse, st, _ = run_attn(wl)
    ref_out, ref_lse, ref_st = oracle_attn(wl)
    assert np.array_equal(st, ref_st)
    compare(wl, out, lse, ref_out, ref_lse, range(wl.B))
    # a root with no context sees only itself: its output is its own value, exactly representable
    r = int(wl.node_offset[2])
    np.testing.assert_allclose(out[r], np.repeat(W.bf16_bits_to_f32(wl.v_node[r]), 4, axis=0), rtol=0, atol=1e-6)


def test_attention_gqa_groups_and_wide_group():
    # G = 16 query heads per kv head: 64 nodes x 16 = 1024 rows = 16 row groups
    rng = np.random.default_rng(12)
    parents = [W.random_tree(rng, 64), W.chain(7)]
    wl = W.make_attn(parents, [300, 129], Hq=16, Hkv=1, seed=13, name="attn_g16")
    for split in (None, 128):
        out, lse, st, _ = run_attn(wl, split=split)
        ref_out, ref_lse, _ = oracle_attn(wl)
        compare(wl, out, lse, ref_out, ref_lse, range(wl.B))


def test_attention_full_size_every_request():
    """The batch-256 shape the benchmark times, in both launch modes (one pass and contexts
    split at 1024 keys): every request against the oracle, one request per task over a pool of
    oracle processes (~200 s of single-core oracle work)."""
    import oracle_pool as OP
    wl = W.make_attn_mixed_b256(0)
    results = {}
    for i, split in enumerate((None, 1024)):
        out, lse, st, _ = run_attn(wl, split=split)
        assert (st == 0).all()
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        results[f"out_{i}"], results[f"lse_{i}"] = out, lse
    arrays = dict(q=wl.q, k_ctx=wl.k_ctx, v_ctx=wl.v_ctx, k_node=wl.k_node, v_node=wl.v_node,
                  node_offset=wl.node_offset, ctx_offset=wl.ctx_offset, parent=wl.parent,
                  scale=np.float64(wl.scale), **results)
    del results
    rows = OP.run(arrays, OP.attention_request, list(range(wl.B)))
    assert sorted(r[0] for r in rows) == list(range(wl.B))
    for i, name in enumerate(("one pass", "split 1024")):
        eo = max(r[1][i][0] for r in rows if r[1])
        el = max(r[1][i][1] for r in rows if r[1])
        print(f"attention batch-256 {name}: all {wl.B} requests, out rel err {eo:.2e}, lse abs err {el:.2e}")
        assert eo <= ATTN_TOL and el <= ATTN_TOL
        assert eo <= ATTN_ENVELOPE and el <= ATTN_ENVELOPE


def _many_small_requests(B, seed):
    """B requests of 0-3 draft nodes (chains or roots) over 0-130 context keys."""
    rng = np.random.default_rng(seed)
    parents, ctx = [], []
    for b in range(B):
        n = int(rng.integers(0, 4))
        parents.append(W.chain(n) if rng.integers(0, 2) else np.full(n, -1, np.int32))
        ctx.append(int(rng.integers(0, 131)))
    return W.make_attn(parents, ctx, Hq=4, Hkv=2, seed=seed, name=f"attn_many{B}")


def test_attention_more_requests_than_the_schedule_holds():
    # 1100 (request, part) items exceed the in-LDS unit list: one workgroup per unit
    wl = _many_small_requests(1100, 31)
    out, lse, st, _ = run_attn(wl, max_nodes=4)
    ref_out, ref_lse, ref_st = oracle_attn(wl, max_nodes=4)
    assert np.array_equal(st, ref_st)
    compare(wl, out, lse, ref_out, ref_lse, range(wl.B))


def test_attention_scheduled_and_per_unit_launches_agree():
    # one pass: 600 items, scheduled list; split 64: 600 x 3 items, one workgroup per unit
    wl = _many_small_requests(600, 32)
    o1, l1, s1, _ = run_attn(wl, max_nodes=4)
    o2, l2, s2, _ = run_attn(wl, max_nodes=4, split=64)
    ref_out, ref_lse, ref_st = oracle_attn(wl, max_nodes=4)
    assert np.array_equal(s1, ref_st) and np.array_equal(s2, ref_st)
    compare(wl, o1, l1, ref_out, ref_lse, range(wl.B))
    compare(wl, o2, l2, ref_out, ref_lse, range(wl.B))


@pytest.mark.parametrize("split", [None, 64])
def test_attention_128_row_units_match_64_row_units(split):
    # trees of at most 16 nodes at 4 query heads per kv head: max_nodes = 16 gives
    # 64-row units staged through registers; max_nodes = 64 gives 128-row units
    # staged by direct loads into two LDS buffers, whose units of <= 64 rows run
    # the same one-tile products, so the outputs must agree bit for bit
    rng = np.random.default_rng(41)
    parents = [W.chain(3), W.root_branch(), W.random_tree(rng, 16), np.array([-1, -1, 0], np.int32),
               W.random_tree(rng, 9), W.chain(16), np.zeros(0, np.int32), W.random_tree(rng, 12)]
    wl = W.make_attn(parents, [0, 1, 63, 64, 65, 200, 7, 517], Hq=8, Hkv=2, seed=41, name="attn_rows")
    o64, l64, s64, _ = run_attn(wl, split=split, max_nodes=16)
    o128, l128, s128, _ = run_attn(wl, split=split, max_nodes=64)
    ref_out, ref_lse, ref_st = oracle_attn(wl, max_nodes=16)
    assert np.array_equal(s64, ref_st) and np.array_equal(s128, ref_st)
    rows = rows_of(wl, range(wl.B))
    assert np.array_equal(o64[rows].view(np.uint32), o128[rows].view(np.uint32))
    assert np.array_equal(l64[rows].view(np.uint32), l128[rows].view(np.uint32))
    compare(wl, o128, l128, ref_out, ref_lse, range(wl.B))


def test_attention_split_chosen_by_the_library():
    # one request, 8 kv heads, a 4096-token context: split = 0 takes 32 parts of 128 keys
    wl = W.make_attn([W.root_branch()], [4096], Hq=32, Hkv=8, seed=5, name="attn_b1")
    o0, l0, s0, _ = run_attn(wl, split=0)
    o1, l1, s1, _ = run_attn(wl, split=128)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)) and np.array_equal(l0.view(np.uint32), l1.view(np.uint32))
    ref_out, ref_lse, ref_st = oracle_attn(wl)
    assert np.array_equal(s0, ref_st)
    compare(wl, o0, l0, ref_out, ref_lse, range(wl.B))
    # the edge mix (8 requests, 2 kv heads, 4 row groups of 64: 64 units, contexts up to 200
    # keys): min(8, 32, 4) = 4 parts of 64 keys
    wl = W.make_attn_small(6)
    o0, l0, s0, _ = run_attn(wl, split=0)
    o1, l1, s1, _ = run_attn(wl, split=64)
    rows = rows_of(wl, range(wl.B))
    assert np.array_equal(o0[rows].view(np.uint32), o1[rows].view(np.uint32)) and np.array_equal(s0, s1)


def test_attention_deterministic():
    wl = W.make_attn_small(5)
    o1, l1, _, d = run_attn(wl, split=64)
    o2, l2, _, _ = run_attn(wl, split=64)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("split", [None, 50])
def test_attention_device_errors(split):
    # request 0 ok, 1 bad mask, 2 context longer than max_ctx, 3 too many nodes, 4 bad node offsets
    parents = [W.chain(3), W.chain(3), W.chain(2), np.full(66, -1, np.int32), W.chain(2)]
    wl = W.make_attn(parents, [40, 40, 120, 10, 10], Hq=4, Hkv=2, seed=21, name="attn_err")
    d = upload_attn(wl)
    anc, _ = G.ancestry(d["node_offset"], d["parent"], max_nodes=64)
    a = anc_u64(anc).copy()
    a[wl.node_offset[1] + 1] = 0b100            # node 1 of request 1 lacks its own bit
    anc_bad = torch.from_numpy(a.view(np.int64)).to(anc.device)
    no = wl.node_offset.copy()
    no_t = torch.from_numpy(no).to(anc.device)
    no_t[5] = no_t[4] - 1                        # request 4 ends before it starts
    out = torch.full((wl.T, wl.Hq, 128), 7.0, device=anc.device)
    o, l, st = G.attention(d["q"], d["k_ctx"], d["v_ctx"], d["ctx_offset"], d["k_node"], d["v_node"], no_t,
                           anc_bad, wl.scale, max_nodes=64, max_ctx=100, split=split, out=out)
    torch.cuda.synchronize()
    st, o = host(st), host(o)
    assert list(st) == [0, A.STATUS_BAD_MASK, A.STATUS_BAD_CONTEXT, O.STATUS_TOO_MANY_NODES, O.STATUS_BAD_OFFSETS]
    for b in (1, 2, 3):
        assert np.isnan(o[wl.node_offset[b]:wl.node_offset[b + 1]]).all()
    assert (o[wl.node_offset[4]:] == 7.0).all()          # bad offsets: untouched
    ref_out, ref_lse, _ = oracle_attn(wl, requests={0}, max_nodes=64, max_ctx=100)
    compare(wl, o, host(l), ref_out, ref_lse, [0])


def test_attention_host_errors():
    wl = W.make_attn_small(0)
    d = upload_attn(wl)
    anc, _ = G.ancestry(d["node_offset"], d["parent"], max_nodes=64)
    args = (d["q"], d["k_ctx"], d["v_ctx"], d["ctx_offset"], d["k_node"], d["v_node"], d["node_offset"], anc)
    with pytest.raises(G.GdnTreeError) as e:
        G.attention(*args, float("nan"), max_nodes=64, max_ctx=wl.max_ctx)
    assert e.value.code == -2
    ws = torch.empty((16,), dtype=torch.uint8, device=anc.device)
    with pytest.raises(G.GdnTreeError) as e:
        G.attention(*args, wl.scale, max_nodes=64, max_ctx=wl.max_ctx, split=32, workspace=ws)
    assert e.value.code == -8


@pytest.mark.parametrize("split", [None, 100])
def test_attention_non_finite_node_values_stay_in_their_subtree(split):
    """TreeWY, Method: a node's row reads its own path only.  NaN and Inf in the keys and values of
    some nodes leave every row that does not see them bit-identical; a row that sees one is
    non-finite exactly where the oracle is, and its other columns meet the bar.  Cases: key groups
    (small units), the plain one-tile layout, 64-node trees, and the split context."""
    import copy
    base = W.make_attn_small(5)
    out0, lse0, st0, _ = run_attn(base, split=split)
    wl = copy.deepcopy(base)
    hit = []   # (request, node) perturbed
    for b in range(wl.B):
        n = int(wl.node_offset[b + 1] - wl.node_offset[b])
        if n >= 2:
            j = n - 1 if b % 2 else n // 2
            t = int(wl.node_offset[b]) + j
            wl.v_node[t, 0, 3] = 0x7F80       # +Inf, kv head 0, column 3
            wl.v_node[t, -1, 100] = 0x7FC0    # NaN, last kv head, column 100
            wl.k_node[t, 0, 7] = 0x7FC0       # NaN key entry: only rows that see the node score it
            hit.append((b, j))
    out1, lse1, st1, _ = run_attn(wl, split=split)
    assert np.array_equal(st0, st1)
    seen = np.zeros(wl.T, bool)
    for b, j in hit:
        lo = int(wl.node_offset[b])
        anc = O.ancestry(wl.parent[lo:int(wl.node_offset[b + 1])])
        for t, m in enumerate(anc):
            seen[lo + t] |= bool((m >> j) & 1)
    rows = rows_of(wl, range(wl.B))
    unseen = rows[~seen[rows]]
    assert np.array_equal(out0[unseen].view(np.uint32), out1[unseen].view(np.uint32))
    assert np.array_equal(lse0[unseen].view(np.uint32), lse1[unseen].view(np.uint32))
    with np.errstate(invalid="ignore", over="ignore"):
        ref_out, ref_lse, _ = oracle_attn(wl)
    inside = rows[seen[rows]]
    got, want = out1[inside].astype(np.float64), ref_out[inside]
    assert np.array_equal(np.isfinite(got), np.isfinite(want))
    fin = np.isfinite(want)
    scale = np.abs(np.where(fin, want, 0)).max(axis=-1, keepdims=True)
    assert (np.abs(np.where(fin, got - want, 0)) / np.maximum(scale, 1e-30)).max() <= ATTN_TOL
