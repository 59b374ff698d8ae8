"""Plain fp64 definition of ancestry-masked (tree-bias) decode attention.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library and imports nothing from it.

What is computed, and where it is defined
-----------------------------------------
GDN Tree-Scan (English abstract): in one target pass over a draft tree, the
attention layers of the model need only an ancestry mask, applied through
FlashAttention-2 tree-bias attention; the recurrent layers are the GDN part.
Read plainly, the row of draft node t sees exactly what sequential decode of
its root-to-node path would see: every token of the request's committed
context, then the draft nodes on its path (its inclusive ancestors, TreeWY
"Method": a branch refers to its common ancestors, never to another branch).
For query head h (key/value head h // (Hq / Hkv), grouped-query heads)::

    keys   = [k_ctx[0 .. Lc) ; k_node[j] for j in anc*(t)]     (same for values)
    s_j    = scale * (q_t,h . key_j)
    lse    = log sum_j exp(s_j)
    out_t,h = sum_j exp(s_j - lse) * value_j

The scale is an argument (1/sqrt(d) in the usual layer).  Each output is the
definition written out: no blocking, no online rescaling, no reordering.

Parity status: see ``PINS`` below.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .gdn_oracle import (STATUS_OK, STATUS_BAD_OFFSETS, STATUS_TOO_MANY_NODES, STATUS_BAD_PARENT,
                         MAX_NODES, ancestry, parents_valid)

__all__ = ["STATUS_BAD_CONTEXT", "STATUS_BAD_MASK", "attention_row", "tree_attention_request",
           "tree_attention_batch", "request_status", "PINS"]

# Status codes of the attention entry point beyond the shared ones (the C-ABI
# header lists the same numbers).
STATUS_BAD_CONTEXT = 7   # ctx_offset not monotone, beyond C, or Lc > max_ctx
STATUS_BAD_MASK = 8      # an ancestry bitset that is not a tree node's (device input only)

PINS = {
    "attention_row": "hand example with closed-form output and lse; q = 0 gives the mean of the "
                     "visible values; one visible key gives its value",
    "tree_attention_request": "equals torch's causal scaled_dot_product_attention (float64, grouped "
                              "heads) over [context, root-to-node path] for every node; non-ancestor "
                              "keys and values do not matter, ancestor ones do",
    "tree_attention_batch": "request independence under permutation; statuses on hand-built bad inputs",
    "request_status": "hand-built bad offsets / contexts / node counts / parents",
}


def attention_row(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """Softmax attention of one query over explicit key/value rows (fp64).

    q [d], keys [n, d], values [n, d_v] with n >= 1.  Returns (out [d_v], lse)."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    s = scale * (keys @ q)
    smax = np.max(s)
    lse = float(smax + np.log(np.sum(np.exp(s - smax))))
    p = np.exp(s - lse)
    return p @ values, lse


def tree_attention_request(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, k_node: np.ndarray,
                           v_node: np.ndarray, parent: Sequence[int], scale: float):
    """One request: q [N][Hq][d], k_ctx/v_ctx [Lc][Hkv][d], k_node/v_node [N][Hkv][d],
    parent [N] (request-local, -1 = root).  Returns out [N][Hq][d], lse [N][Hq]."""
    N, Hq, d = q.shape
    Hkv = k_node.shape[1] if N else k_ctx.shape[1]
    G = Hq // Hkv
    anc = ancestry(parent)
    out = np.zeros((N, Hq, v_node.shape[2] if N else d))
    lse = np.zeros((N, Hq))
    for t in range(N):
        nodes = [j for j in range(N) if (anc[t] >> j) & 1]
        for h in range(Hq):
            hk = h // G
            keys = np.concatenate([np.asarray(k_ctx[:, hk], np.float64), np.asarray(k_node[nodes, hk], np.float64)])
            vals = np.concatenate([np.asarray(v_ctx[:, hk], np.float64), np.asarray(v_node[nodes, hk], np.float64)])
            out[t, h], lse[t, h] = attention_row(q[t, h], keys, vals, scale)
    return out, lse


def request_status(node_offset, ctx_offset, b: int, T: int, C: int, max_nodes: int, max_ctx: int,
                   parent) -> int:
    """Per-request status, checked in this order: node offsets, node count,
    context offsets and length, tree (parent-before-child)."""
    lo, hi = int(node_offset[b]), int(node_offset[b + 1])
    if lo < 0 or hi < lo or hi > T:
        return STATUS_BAD_OFFSETS
    if hi - lo > min(max_nodes, MAX_NODES):
        return STATUS_TOO_MANY_NODES
    c0, c1 = int(ctx_offset[b]), int(ctx_offset[b + 1])
    if c0 < 0 or c1 < c0 or c1 > C or c1 - c0 > max_ctx:
        return STATUS_BAD_CONTEXT
    if not parents_valid(parent[lo:hi]):
        return STATUS_BAD_PARENT
    return STATUS_OK


def tree_attention_batch(q, k_ctx, v_ctx, ctx_offset, k_node, v_node, node_offset, parent, Hq: int,
                         Hkv: int, scale: float, max_nodes: int = MAX_NODES, max_ctx: int = 1 << 30,
                         requests=None):
    """Whole batch.  q [T][Hq][d]; k_ctx, v_ctx [C][Hkv][d]; k_node, v_node [T][Hkv][d];
    ctx_offset, node_offset [B+1]; parent [T].  Returns (out [T][Hq][d], lse [T][Hq],
    status [B]).  Rows of a request with a bad status are NaN (bad offsets: untouched NaN)."""
    T = q.shape[0]
    C = k_ctx.shape[0]
    B = len(node_offset) - 1
    out = np.full((T, Hq, q.shape[2]), np.nan)
    lse = np.full((T, Hq), np.nan)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        st = request_status(node_offset, ctx_offset, b, T, C, max_nodes, max_ctx, parent)
        status[b] = st
        if st != STATUS_OK or (requests is not None and b not in requests):
            continue
        lo, hi = int(node_offset[b]), int(node_offset[b + 1])
        c0, c1 = int(ctx_offset[b]), int(ctx_offset[b + 1])
        if hi == lo:
            continue
        o, l = tree_attention_request(q[lo:hi], k_ctx[c0:c1], v_ctx[c0:c1], k_node[lo:hi], v_node[lo:hi],
                                      parent[lo:hi], scale)
        out[lo:hi] = o
        lse[lo:hi] = l
    return out, lse, status
