"""Plain, slow fp64 definition of tree-structured GDN speculative verification.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library and imports nothing from it.

What is computed, and where it is defined
-----------------------------------------
* The gated delta rule, one decode step (GDN's update, as TreeWY's abstract and
  "Background" describe GDN layers: a fixed-size recurrent state per head)::

      alpha = exp(g);   u = beta * (v - alpha * S k);   S' = alpha * S + u k^T;   o = S' q

  S is the d_v x d_k state in math orientation; the device stores it
  transposed, H = S^T, as [d_k][d_v].  ``u`` is the pseudo-value with beta
  folded in: the new value minus what the decayed preceding state already
  predicts for this key (TreeWY, "Method").
* Tree semantics (GDN Tree-Scan, English abstract): every draft node's row
  must see the recurrent state that plain sequential decode produces along its
  root-to-node path.  The oracle therefore walks nodes in parent-before-child
  order (TreeWY, "Method") and applies the step to the parent's state; a node
  with parent -1 starts from the committed state S0.  Nothing is shared between
  branches except common ancestors (TreeWY, "Method": a branch refers to its
  common ancestors, never to the other branch).
* Commit (TreeWY, "Method" and "Novelty"; Tree-Scan: accepted-chain-only state
  publication): the next committed state is the sequential state at the last
  node of the accepted root-first path; an empty path keeps S0.
* storeall (TreeWY, "Prior work": vLLM's default keeps the committed state and
  one state per candidate position and selects the accepted one): node_state[t]
  is the state after node t, and its commit copies the accepted node's state.

There is no blocking, reordering or algebraic rewrite here: the tree-WY
identities that the HIP kernels use are checked against this file, not used
by it.

Parity status of each function: see the module-level ``PINS`` table.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "STATUS_OK", "STATUS_BAD_OFFSETS", "STATUS_TOO_MANY_NODES", "STATUS_BAD_PARENT",
    "STATUS_BAD_PATH", "STATUS_BAD_ACCEPT", "STATUS_BAD_SLOT", "MAX_NODES",
    "parents_valid", "ancestry", "depths", "root_to_node", "accepted_path", "gated_delta_step",
    "verify_unit", "commit_unit", "replay_commit_unit", "verify_request", "verify_batch",
    "commit_batch", "accepted_path_batch", "verify_storeall_batch", "commit_storeall_batch",
    "state_bytes", "PINS", "greedy_accept", "greedy_accept_batch", "survival", "budget_select",
]

# Status codes written per request.  These numbers are part of the C-ABI's
# interface (its header lists the same values), not shared code.
STATUS_OK = 0
STATUS_BAD_OFFSETS = 1      # node_offset not monotone or beyond T
STATUS_TOO_MANY_NODES = 2   # N_b > max_nodes (or > 64)
STATUS_BAD_PARENT = 3       # parent[t] >= t or < -1
STATUS_BAD_PATH = 4         # path is not a root-first chain of the request's tree
STATUS_BAD_ACCEPT = 5       # accept_node outside [-1, N_b)
STATUS_BAD_SLOT = 6         # state_slot[b] outside [0, n_slots)

MAX_NODES = 64

# Which independent check pins each function (tests/test_oracle_pins.py).
PINS = {
    "ancestry": "brute-force parent walk; chain closed form; pages' two-branch example",
    "depths": "equals popcount of ancestry; chain closed form",
    "accepted_path": "chain structure (root parent -1, consecutive parents, ends at node)",
    "gated_delta_step": "finite-difference gradient of the least-squares loss; delta-rule "
                        "write property; orthogonal-complement decay; alpha=0 and beta=0 "
                        "closed forms; storage-layout definition",
    "verify_unit": "brute-force replay of every root-to-node path; sibling invariance; "
                   "relabelling; independent tree-WY triangular-solve formulation",
    "commit_unit": "equals the accepted node's sequential state; empty path keeps S0; "
                   "verify-then-commit composition",
    "verify_storeall_batch": "node states equal the per-path sequential states; state count "
                             "of a depth-3 chain is 4 including S0 (TreeWY, Prior work)",
    "survival": "equals the running product over each explicit root-to-node path; chain closed form",
    "budget_select": "order property (every kept node outranks every dropped one), ancestor closure, "
                     "count = min(budget, nodes at or above the threshold), threshold respected",
    "greedy_accept": "brute force over every root-first path: with distinct sibling tokens the "
                     "result is the longest path whose every token matches the target's "
                     "prediction at its parent; a chain accepts exactly its matching prefix",
}


# ----------------------------------------------------------------------------
# tree structure
# ----------------------------------------------------------------------------

def parents_valid(parent: Sequence[int]) -> bool:
    """Parent-before-child order: every parent index is -1 or an earlier node."""
    return all(-1 <= int(p) < i for i, p in enumerate(parent))


def ancestry(parent: Sequence[int]) -> List[int]:
    """Inclusive ancestor set of each node as a bitmask (bit j = node j).

    anc(t) = anc(parent(t)) | {t}, with anc(-1) empty (TreeWY, "Method";
    Tree-Scan's ancestry mask).  Requires a valid parent array.
    """
    anc: List[int] = []
    for t, p in enumerate(parent):
        p = int(p)
        anc.append((anc[p] if p >= 0 else 0) | (1 << t))
    return anc


def depths(parent: Sequence[int]) -> List[int]:
    """Depth of each node; a node attached to S0 has depth 1."""
    out: List[int] = []
    for p in parent:
        p = int(p)
        out.append(1 if p < 0 else out[p] + 1)
    return out


def root_to_node(parent: Sequence[int], t: int) -> List[int]:
    """The node indices from the S0-attached root down to t, inclusive."""
    path = []
    while t >= 0:
        path.append(t)
        t = int(parent[t])
    return path[::-1]


def accepted_path(parent: Sequence[int], accept_node: int) -> List[int]:
    """Root-first accepted path ending at accept_node; [] when none is accepted."""
    if accept_node < 0:
        return []
    return root_to_node(parent, accept_node)


# ----------------------------------------------------------------------------
# the sequential rule
# ----------------------------------------------------------------------------

def gated_delta_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     g: float, beta: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One gated-delta-rule decode step in fp64.

    S is d_v x d_k (math orientation).  Returns (S_new, u, o) where u is the
    pseudo-value (beta folded in) and o the output read from the updated state.
    """
    alpha = math.exp(float(g))
    u = float(beta) * (v - alpha * (S @ k))
    S_new = alpha * S + np.outer(u, k)
    o = S_new @ q
    return S_new, u, o


def verify_unit(H0: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                g: np.ndarray, beta: np.ndarray, parent: Sequence[int]):
    """One (request, v-head) unit.

    H0: [d_k][d_v] stored state.  q, k: [N][d_k]; v: [N][d_v]; g, beta: [N].
    Returns (O [N][d_v], U [N][d_v], states) where states[t] is the math-
    orientation state after node t.
    """
    S_root = np.ascontiguousarray(np.asarray(H0, np.float64).T)
    N = len(parent)
    dv = S_root.shape[0]
    O = np.zeros((N, dv))
    U = np.zeros((N, dv))
    states: List[np.ndarray] = []
    for t in range(N):
        p = int(parent[t])
        P = S_root if p < 0 else states[p]
        S_t, u_t, o_t = gated_delta_step(P, q[t], k[t], v[t], g[t], beta[t])
        states.append(S_t)
        U[t] = u_t
        O[t] = o_t
    return O, U, states


def commit_unit(H0: np.ndarray, states: List[np.ndarray], path: Sequence[int]) -> np.ndarray:
    """Next committed state in storage orientation: the accepted node's state,
    or S0 unchanged when the path is empty."""
    if len(path) == 0:
        return np.asarray(H0, np.float64).copy()
    return states[int(path[-1])].T.copy()


def replay_commit_unit(H0, q, k, v, g, beta, path: Sequence[int]) -> np.ndarray:
    """Committed state by replaying the accepted path from S0 with the
    sequential rule (ReplaySSM / Tree-Scan's branch replay).  Storage orientation."""
    S = np.ascontiguousarray(np.asarray(H0, np.float64).T)
    for t in path:
        S, _, _ = gated_delta_step(S, q[t], k[t], v[t], g[t], beta[t])
    return S.T.copy()


# ----------------------------------------------------------------------------
# batch wrappers mirroring the C-ABI layouts
# ----------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _request_status(node_offset, b, T, max_nodes, parent, slot=0, n_slots=1) -> int:
    """Checks in a fixed order: offsets, node count, parent order, state slot."""
    lo, hi = int(node_offset[b]), int(node_offset[b + 1])
    if lo < 0 or hi < lo or hi > T:
        return STATUS_BAD_OFFSETS
    if hi - lo > min(max_nodes, MAX_NODES):
        return STATUS_TOO_MANY_NODES
    if not parents_valid(parent[lo:hi]):
        return STATUS_BAD_PARENT
    if not 0 <= slot < n_slots:
        return STATUS_BAD_SLOT
    return STATUS_OK


def _slot(state_slot, b):
    return b if state_slot is None else int(state_slot[b])


def verify_request(S0, q, k, v, g, beta, node_offset, parent, b: int, Hv: int, Hk: int,
                   max_nodes: int = MAX_NODES, state_slot=None, heads=None):
    """All v-heads (or the listed ones) of request b.

    Returns (status, O [N][Hv][d], U [N][Hv][d], anc list, states) where
    states[h] is the list of node states of head h (math orientation).
    Arrays are float64 views of the device inputs (q, k, v already widened).
    """
    T = len(parent)
    slot = _slot(state_slot, b)
    st = _request_status(node_offset, b, T, max_nodes, parent, slot, S0.shape[0])
    lo, hi = int(node_offset[b]), int(node_offset[b + 1])
    if st != STATUS_OK:
        return st, None, None, None, None
    par = [int(p) for p in parent[lo:hi]]
    N = hi - lo
    d_v = S0.shape[-1]
    r = Hv // Hk
    O = np.zeros((N, Hv, d_v))
    U = np.zeros((N, Hv, d_v))
    states = {}
    for h in (range(Hv) if heads is None else heads):
        hk = h // r
        o, u, s = verify_unit(_f64(S0[slot, h]), q[lo:hi, hk], k[lo:hi, hk], v[lo:hi, h],
                              _f64(g[lo:hi, h]), _f64(beta[lo:hi, h]), par)
        O[:, h] = o
        U[:, h] = u
        states[h] = s
    return st, O, U, ancestry(par), states


def verify_batch(S0, q, k, v, g, beta, node_offset, parent, Hv: int, Hk: int,
                 max_nodes: int = MAX_NODES, state_slot=None):
    """Whole batch: (O [T][Hv][d], U [T][Hv][d], anc uint64 [T], status int32 [B]).

    A request whose status is nonzero gets NaN rows in O and U and zero
    ancestry masks (when its rows are addressable at all).
    """
    T = len(parent)
    B = len(node_offset) - 1
    d_v = S0.shape[-1]
    O = np.zeros((T, Hv, d_v))
    U = np.zeros((T, Hv, d_v))
    anc = np.zeros(T, dtype=np.uint64)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        st, Ob, Ub, ab, _ = verify_request(S0, q, k, v, g, beta, node_offset, parent, b, Hv, Hk,
                                           max_nodes, state_slot)
        status[b] = st
        lo, hi = int(node_offset[b]), int(node_offset[b + 1])
        if st == STATUS_OK:
            O[lo:hi] = Ob
            U[lo:hi] = Ub
            anc[lo:hi] = np.array(ab, dtype=np.uint64)
        elif st != STATUS_BAD_OFFSETS:
            O[lo:hi] = np.nan
            U[lo:hi] = np.nan
    return O, U, anc, status


def _path_status(parent_local: Sequence[int], path: Sequence[int]) -> int:
    N = len(parent_local)
    if len(path) > N:
        return STATUS_BAD_PATH
    prev = -1
    for t in path:
        t = int(t)
        if t < 0 or t >= N or int(parent_local[t]) != prev:
            return STATUS_BAD_PATH
        prev = t
    return STATUS_OK


def commit_batch(S0, q, k, v, g, beta, node_offset, parent, path, path_len, Hv: int, Hk: int,
                 max_nodes: int = MAX_NODES, state_slot=None, S_out_init=None, requests=None):
    """Committed states by definition: the sequential state at each request's
    accepted node, replayed from S0 along the accepted root-first path.

    path: int32 [B][max_nodes] root-first; path_len: int32 [B].  Returns
    (S_out [n_slots][Hv][d_k][d_v] storage orientation, status [B]).  S_out
    starts as a copy of S_out_init (default S0); an invalid request or path
    writes a copy of S0 into its slot, a bad slot writes nothing.  With
    ``requests``, only those requests are evaluated (others keep status 0).
    """
    B = len(node_offset) - 1
    out = np.array(S0 if S_out_init is None else S_out_init, dtype=np.float64, copy=True)
    status = np.zeros(B, dtype=np.int32)
    T = len(parent)
    r = Hv // Hk
    for b in (range(B) if requests is None else requests):
        slot = _slot(state_slot, b)
        st = _request_status(node_offset, b, T, max_nodes, parent, slot, S0.shape[0])
        L = int(path_len[b]) if st == STATUS_OK else 0
        lo, hi = int(node_offset[b]), int(node_offset[b + 1])
        if st == STATUS_OK:
            if L < 0 or L > max_nodes:
                st = STATUS_BAD_PATH
            else:
                st = _path_status(parent[lo:hi], path[b][:L])
        status[b] = st
        if not 0 <= slot < S0.shape[0]:
            continue
        if st != STATUS_OK or L == 0:
            out[slot] = _f64(S0[slot])
            continue
        pth = [int(t) for t in path[b][:L]]
        for h in range(Hv):
            hk = h // r
            out[slot, h] = replay_commit_unit(_f64(S0[slot, h]), q[lo:hi, hk], k[lo:hi, hk],
                                              v[lo:hi, h], _f64(g[lo:hi, h]), _f64(beta[lo:hi, h]), pth)
    return out, status


def accepted_path_batch(node_offset, parent, accept_node, max_nodes: int = MAX_NODES):
    """(path int32 [B][max_nodes] root-first, zero-filled; path_len [B]; status [B])."""
    B = len(node_offset) - 1
    T = len(parent)
    path = np.zeros((B, max_nodes), dtype=np.int32)
    plen = np.zeros(B, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        st = _request_status(node_offset, b, T, max_nodes, parent)
        lo, hi = int(node_offset[b]), int(node_offset[b + 1])
        a = int(accept_node[b])
        if st == STATUS_OK and not (-1 <= a < hi - lo):
            st = STATUS_BAD_ACCEPT
        status[b] = st
        if st != STATUS_OK:
            continue
        p = accepted_path(parent[lo:hi], a)
        plen[b] = len(p)
        path[b, :len(p)] = p
    return path, plen, status


def verify_storeall_batch(S0, q, k, v, g, beta, node_offset, parent, Hv: int, Hk: int,
                          max_nodes: int = MAX_NODES, state_slot=None, requests=None):
    """storeall: (O, node_state [T][Hv][d_k][d_v] storage orientation, status).

    With ``requests`` only those requests are evaluated (others left zero).
    """
    T = len(parent)
    B = len(node_offset) - 1
    d = S0.shape[-1]
    O = np.zeros((T, Hv, d))
    NS = np.zeros((T, Hv, d, d))
    status = np.zeros(B, dtype=np.int32)
    for b in (range(B) if requests is None else requests):
        st, Ob, _, _, states = verify_request(S0, q, k, v, g, beta, node_offset, parent, b, Hv, Hk,
                                              max_nodes, state_slot)
        status[b] = st
        lo, hi = int(node_offset[b]), int(node_offset[b + 1])
        if st == STATUS_OK:
            O[lo:hi] = Ob
            for h, sl in states.items():
                for t, S in enumerate(sl):
                    NS[lo + t, h] = S.T
        elif st != STATUS_BAD_OFFSETS:
            O[lo:hi] = np.nan
    return O, NS, status


def commit_storeall_batch(S0, node_state, node_offset, parent, accept_node, max_nodes: int = MAX_NODES,
                          state_slot=None, S_out_init=None):
    """storeall commit: copy the accepted node's stored state into the request's
    slot (S0 when none is accepted or the request is invalid; nothing on a bad
    slot).  Returns (S_out [n_slots]..., status [B])."""
    B = len(node_offset) - 1
    T = len(parent)
    out = np.array(S0 if S_out_init is None else S_out_init, dtype=np.float64, copy=True)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        slot = _slot(state_slot, b)
        st = _request_status(node_offset, b, T, max_nodes, parent, slot, S0.shape[0])
        lo, hi = int(node_offset[b]), int(node_offset[b + 1])
        a = int(accept_node[b])
        if st == STATUS_OK and not (-1 <= a < hi - lo):
            st = STATUS_BAD_ACCEPT
        status[b] = st
        if not 0 <= slot < S0.shape[0]:
            continue
        out[slot] = _f64(S0[slot]) if (st != STATUS_OK or a < 0) else _f64(node_state[lo + a])
    return out, status


def greedy_accept(parent: Sequence[int], draft: Sequence[int], target_next: Sequence[int],
                  root_next: int) -> int:
    """Greedy tree acceptance (TreeWY, Results: greedy drafting and verification; GDN
    Tree-Scan: the committed draft is chosen on the device).

    Start at the committed root, whose target prediction is root_next.  Among the
    current position's children, in index order, take the first whose draft token
    equals the target's prediction at the current position; continue from it with
    its own prediction target_next[child].  Stop when no child matches.  Returns
    the last accepted node, or -1 when the first level already fails.
    """
    children = {}
    for t, p in enumerate(parent):
        children.setdefault(int(p), []).append(t)
    cur, want = -1, int(root_next)
    while True:
        nxt = next((c for c in children.get(cur, []) if int(draft[c]) == want), None)
        if nxt is None:
            return cur
        cur, want = nxt, int(target_next[nxt])


def greedy_accept_batch(node_offset, parent, draft, target_next, root_next, max_nodes: int = MAX_NODES):
    """(accept_node [B], path [B][max_nodes], path_len [B], status [B]) for a batch."""
    B = len(node_offset) - 1
    T = len(parent)
    acc = np.full(B, -1, dtype=np.int32)
    path = np.zeros((B, max_nodes), dtype=np.int32)
    plen = np.zeros(B, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        st = _request_status(node_offset, b, T, max_nodes, parent)
        status[b] = st
        if st != STATUS_OK:
            continue
        lo, hi = int(node_offset[b]), int(node_offset[b + 1])
        a = greedy_accept(parent[lo:hi], draft[lo:hi], target_next[lo:hi], root_next[b])
        acc[b] = a
        pth = accepted_path(parent[lo:hi], a)
        plen[b] = len(pth)
        path[b, :len(pth)] = pth
    return acc, path, plen, status


def survival(parent: Sequence[int], p: Sequence[float]) -> np.ndarray:
    """Probability that the draft survives verification down to each node: the
    product of the acceptance probabilities along its root-to-node path (DSpark
    adaptive verification: per-token acceptance, then per-position survival;
    TreeSpark: a branch's value is the product of calibrated estimates along it).
    Computed in float32, root first: s_t = s_parent(t) * p_t, so that a device
    making the same fp32 products takes the same selection decisions."""
    s = np.zeros(len(parent), dtype=np.float32)
    for t, par in enumerate(parent):
        pt = np.float32(p[t])
        s[t] = pt if int(par) < 0 else np.float32(s[int(par)] * pt)
    return s


def budget_select(node_offset, parent, p, budget: int, threshold: float, max_nodes: int = MAX_NODES):
    """Load-adaptive choice of the nodes to verify (DSpark: a global budget B is
    given to the positions with the highest survival across requests; TreeSpark:
    growth stops when the best remaining value is below a threshold).

    Order: survival descending, then depth ascending, then global node index
    ascending (a total order in which every ancestor precedes its descendants,
    survival never increasing along a path).  Keep the first `budget` nodes of
    the valid requests, then drop those with survival below `threshold`.
    Returns (survival f32 [T] (NaN for invalid requests), keep u8 [T],
    kept_per_request i32 [B], status i32 [B]).
    """
    B = len(node_offset) - 1
    T = len(parent)
    surv = np.full(T, np.nan, dtype=np.float32)
    keep = np.zeros(T, dtype=np.uint8)
    status = np.zeros(B, dtype=np.int32)
    cand = []
    for b in range(B):
        st = _request_status(node_offset, b, T, max_nodes, parent)
        status[b] = st
        if st != STATUS_OK:
            continue
        lo, hi = int(node_offset[b]), int(node_offset[b + 1])
        sb = survival(parent[lo:hi], p[lo:hi])
        dep = depths(parent[lo:hi])
        surv[lo:hi] = sb
        cand += [(-float(sb[t]), dep[t], lo + t) for t in range(hi - lo)]
    cand.sort()
    for _, _, gt in cand[:max(0, int(budget))]:
        if surv[gt] >= np.float32(threshold):
            keep[gt] = 1
    counts = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if status[b] == STATUS_OK:
            counts[b] = int(keep[int(node_offset[b]):int(node_offset[b + 1])].sum())
    return surv, keep, counts, status


def state_bytes(B: int, Hv: int, d_k: int, d_v: int, T: int, storeall: bool) -> int:
    """Speculative recurrent-state memory of one layer, excluding S0.

    storeall keeps one fp32 d_k x d_v state per (node, head) (TreeWY, "Prior
    work"); the tree-WY path keeps the fp32 pseudo-value matrix U, one d_v row
    per (node, head) (TreeWY, "Novelty": a small pseudo-value matrix instead of
    per-node states).
    """
    if storeall:
        return T * Hv * d_k * d_v * 4
    return T * Hv * d_v * 4
