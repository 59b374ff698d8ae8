"""Pins of the tree-bias attention oracle against facts that do not come from it.

* a hand example whose output and log-sum-exp are closed forms;
* q = 0 gives the plain mean of the visible values; one visible key gives its value;
* every node's row equals torch's causal scaled_dot_product_attention (float64,
  grouped heads) over [context, root-to-node path]: the attention a sequential
  decoder of that path computes (GDN Tree-Scan, English abstract: the attention
  layers need only an ancestry mask);
* keys and values of non-ancestors do not change a row, an ancestor's do;
* requests are independent (a permutation of requests permutes the rows);
* statuses on hand-built bad inputs.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import gdn_oracle as O
from oracle import tree_attention as A


def test_hand_example_closed_form():
    # scores 0 and ln 3 -> weights 1/4, 3/4; values 4 and 8 -> 7; lse = ln 4
    q = np.array([1.0])
    keys = np.array([[0.0], [math.log(3.0)]])
    vals = np.array([[4.0], [8.0]])
    out, lse = A.attention_row(q, keys, vals, 1.0)
    assert out[0] == pytest.approx(7.0, rel=1e-15)
    assert lse == pytest.approx(math.log(4.0), rel=1e-15)


def test_zero_query_is_mean_and_single_key_is_value():
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((9, 16))
    vals = rng.standard_normal((9, 16))
    out, lse = A.attention_row(np.zeros(16), keys, vals, 0.25)
    np.testing.assert_allclose(out, vals.mean(0), rtol=1e-13, atol=1e-15)
    assert lse == pytest.approx(math.log(9.0), rel=1e-14)
    q = rng.standard_normal(16)
    out, lse = A.attention_row(q, keys[:1], vals[:1], 0.5)
    np.testing.assert_array_equal(out, vals[0])
    assert lse == pytest.approx(0.5 * float(keys[0] @ q), rel=1e-14)


def _sdpa_path(wl, b, t):
    """torch SDPA of node t's path queries over [context, path], returned for the last position."""
    lo = int(wl.node_offset[b])
    c0, c1 = int(wl.ctx_offset[b]), int(wl.ctx_offset[b + 1])
    par = wl.parent[lo:int(wl.node_offset[b + 1])]
    path = O.root_to_node(par, t)
    Lc = c1 - c0
    to64 = lambda x: torch.from_numpy(W.bf16_bits_to_f32(x).astype(np.float64))
    kc, vc = to64(wl.k_ctx[c0:c1]), to64(wl.v_ctx[c0:c1])          # [Lc][Hkv][d]
    kn, vn = to64(wl.k_node[lo + np.array(path)]), to64(wl.v_node[lo + np.array(path)])
    qp = to64(wl.q[lo + np.array(path)])                            # [P][Hq][d]
    keys = torch.cat([kc, kn]).permute(1, 0, 2).unsqueeze(0)        # [1][Hkv][Lc+P][d]
    vals = torch.cat([vc, vn]).permute(1, 0, 2).unsqueeze(0)
    P = len(path)
    # queries sit at positions Lc .. Lc+P-1; a boolean mask lets position i see keys <= i
    qq = qp.permute(1, 0, 2).unsqueeze(0)                           # [1][Hq][P][d]
    pos = torch.arange(Lc, Lc + P).unsqueeze(1)
    mask = torch.arange(Lc + P).unsqueeze(0) <= pos                 # [P][Lc+P]
    o = F.scaled_dot_product_attention(qq, keys, vals, attn_mask=mask, scale=wl.scale, enable_gqa=True)
    return o[0, :, -1, :].numpy()                                   # [Hq][d]


@pytest.mark.parametrize("seed", [0, 1])
def test_rows_equal_sequential_causal_attention(seed):
    wl = W.make_attn_small(seed)
    out, lse, status = A.tree_attention_batch(
        W.bf16_bits_to_f32(wl.q).astype(np.float64), W.bf16_bits_to_f32(wl.k_ctx), W.bf16_bits_to_f32(wl.v_ctx),
        wl.ctx_offset, W.bf16_bits_to_f32(wl.k_node), W.bf16_bits_to_f32(wl.v_node), wl.node_offset, wl.parent,
        wl.Hq, wl.Hkv, wl.scale)
    assert (status == 0).all()
    rng = np.random.default_rng(seed)
    for b in range(wl.B):
        lo, hi = int(wl.node_offset[b]), int(wl.node_offset[b + 1])
        ts = list(range(hi - lo)) if hi - lo <= 6 else sorted(rng.choice(hi - lo, 6, replace=False))
        for t in ts:
            ref = _sdpa_path(wl, b, int(t))
            np.testing.assert_allclose(out[lo + t], ref, rtol=1e-10, atol=1e-12)


def test_non_ancestors_do_not_matter_ancestors_do():
    par = np.array([-1, 0, 0, 1, 2], np.int32)      # node 3 sees {0, 1, 3}; nodes 2, 4 are off its path
    wl = W.make_attn([par], [5], Hq=4, Hkv=2, seed=5)
    f = lambda x: W.bf16_bits_to_f32(x).astype(np.float64)
    args = lambda kn, vn: (f(wl.q), f(wl.k_ctx), f(wl.v_ctx), wl.ctx_offset, kn, vn, wl.node_offset, wl.parent,
                           wl.Hq, wl.Hkv, wl.scale)
    base, _, _ = A.tree_attention_batch(*args(f(wl.k_node), f(wl.v_node)))
    kn, vn = f(wl.k_node), f(wl.v_node)
    kn[[2, 4]] += 3.0
    vn[[2, 4]] -= 5.0
    other, _, _ = A.tree_attention_batch(*args(kn, vn))
    np.testing.assert_array_equal(other[3], base[3])
    np.testing.assert_array_equal(other[1], base[1])
    kn, vn = f(wl.k_node), f(wl.v_node)
    vn[1] += 1.0
    moved, _, _ = A.tree_attention_batch(*args(kn, vn))
    assert np.abs(moved[3] - base[3]).max() > 1e-3
    np.testing.assert_array_equal(moved[2], base[2])


def test_non_finite_values_of_other_branches_do_not_reach_a_row():
    """TreeWY, Method: a node's row sees its own path only.  NaN or Inf in the keys
    and values of nodes off that path leave the row's output and lse bit-identical;
    an Inf in an ancestor's value makes exactly that value column non-finite."""
    par = np.array([-1, 0, 0, 1, 2], np.int32)      # node 3 sees {0, 1, 3}; nodes 2, 4 are off its path
    wl = W.make_attn([par], [5], Hq=4, Hkv=2, seed=5)
    f = lambda x: W.bf16_bits_to_f32(x).astype(np.float64)
    args = lambda kn, vn: (f(wl.q), f(wl.k_ctx), f(wl.v_ctx), wl.ctx_offset, kn, vn, wl.node_offset, wl.parent,
                           wl.Hq, wl.Hkv, wl.scale)
    base, base_lse, _ = A.tree_attention_batch(*args(f(wl.k_node), f(wl.v_node)))
    kn, vn = f(wl.k_node), f(wl.v_node)
    kn[2, :, 5] = np.nan
    vn[2, :, 7] = np.inf
    vn[4, 1, 9] = np.nan
    with np.errstate(invalid="ignore"):
        other, other_lse, _ = A.tree_attention_batch(*args(kn, vn))
    for t in (1, 3):
        np.testing.assert_array_equal(other[t], base[t])
        np.testing.assert_array_equal(other_lse[t], base_lse[t])
    kn, vn = f(wl.k_node), f(wl.v_node)
    vn[1, 0, 7] = np.inf                              # ancestor of node 3, kv head 0 (query heads 0, 1)
    with np.errstate(invalid="ignore"):
        moved, moved_lse, _ = A.tree_attention_batch(*args(kn, vn))
    assert not np.isfinite(moved[3, :2, 7]).any() and np.isfinite(np.delete(moved[3, :2], 7, axis=1)).all()
    np.testing.assert_array_equal(moved[3, 2:], base[3, 2:])
    np.testing.assert_array_equal(moved_lse, base_lse)
    np.testing.assert_array_equal(moved[2], base[2])


def test_requests_are_independent_under_permutation():
    wl = W.make_attn_small(2)
    perm = [3, 0, 7, 1, 6, 2, 5, 4]
    parents = [wl.parent[wl.node_offset[b]:wl.node_offset[b + 1]] for b in range(wl.B)]
    f = lambda x: W.bf16_bits_to_f32(x).astype(np.float64)

    def rows(a, b, off):
        return a[off[b]:off[b + 1]]
    q_p = np.concatenate([rows(wl.q, b, wl.node_offset) for b in perm])
    kn_p = np.concatenate([rows(wl.k_node, b, wl.node_offset) for b in perm])
    vn_p = np.concatenate([rows(wl.v_node, b, wl.node_offset) for b in perm])
    kc_p = np.concatenate([rows(wl.k_ctx, b, wl.ctx_offset) for b in perm])
    vc_p = np.concatenate([rows(wl.v_ctx, b, wl.ctx_offset) for b in perm])
    no = np.concatenate([[0], np.cumsum([len(parents[b]) for b in perm])]).astype(np.int32)
    co = np.concatenate([[0], np.cumsum([int(np.diff(wl.ctx_offset)[b]) for b in perm])]).astype(np.int32)
    par_p = np.concatenate([parents[b] for b in perm]).astype(np.int32)
    base, lse0, _ = A.tree_attention_batch(f(wl.q), f(wl.k_ctx), f(wl.v_ctx), wl.ctx_offset, f(wl.k_node),
                                           f(wl.v_node), wl.node_offset, wl.parent, wl.Hq, wl.Hkv, wl.scale)
    pm, lse1, _ = A.tree_attention_batch(f(q_p), f(kc_p), f(vc_p), co, f(kn_p), f(vn_p), no, par_p,
                                         wl.Hq, wl.Hkv, wl.scale)
    for i, b in enumerate(perm):
        np.testing.assert_array_equal(pm[no[i]:no[i + 1]], rows(base, b, wl.node_offset))
        np.testing.assert_array_equal(lse1[no[i]:no[i + 1]], rows(lse0, b, wl.node_offset))


def test_statuses_on_bad_inputs():
    no = np.array([0, 2, 1, 3, 70], np.int32)
    co = np.array([0, 4, 3, 9, 9], np.int32)
    par = np.array([-1, 0, -1] + [-1] * 67, np.int32)
    T, C = 70, 9
    assert A.request_status(no, co, 0, T, C, 64, 100, par) == O.STATUS_OK
    assert A.request_status(no, co, 1, T, C, 64, 100, par) == O.STATUS_BAD_OFFSETS
    assert A.request_status(no, co, 3, T, C, 64, 100, par) == O.STATUS_TOO_MANY_NODES
    assert A.request_status(no, co, 0, T, C, 64, 3, par) == A.STATUS_BAD_CONTEXT     # Lc 4 > max_ctx 3
    co_bad = np.array([0, 4, 2, 9, 9], np.int32)                                      # decreasing
    assert A.request_status(np.array([0, 1, 2, 3, 4], np.int32), co_bad, 1, T, C, 64, 100, par) == A.STATUS_BAD_CONTEXT
    par_bad = np.array([0, 0, -1] + [-1] * 67, np.int32)                              # parent[0] = 0 >= 0
    assert A.request_status(no, co, 0, T, C, 64, 100, par_bad) == O.STATUS_BAD_PARENT
