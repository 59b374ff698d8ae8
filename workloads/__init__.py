"""Seeded synthetic inputs for tree-structured GDN speculative verification.

This module only draws random inputs: draft-tree shapes, the synthetic
acceptance decision, the committed state S0 and the per-node q, k, v, beta and
gate g.  It holds none of the method's arithmetic (no state update, no solve, no
commit) and it is the one module that both the fp64 oracle's callers and the
HIP path's callers share.

Shapes follow the workloads the TreeWY and GDN Tree-Scan pages run:

* depth-3 draft chains (TreeWY, "Results": depth-3 candidate chains, greedy);
* a 6-node tree of two depth-3 branches off the committed root (GDN Tree-Scan,
  English abstract: "six-node root-branch tree");
* wider random trees and a batch of up to 256 concurrent requests (TreeWY,
  "Results": concurrency 256).

Layouts (all row-major, the same ones the C-ABI takes):

* ``parent``      int32 [T], request-local index of the parent, -1 = attached to S0
* ``node_offset`` int32 [B+1], request b owns rows node_offset[b] .. node_offset[b+1]-1
* ``S0``          float32 [B][Hv][d_k][d_v]  (the state stored transposed: row i
                  is what the state returns for key e_i)
* ``q``, ``k``    bf16 bits (uint16) [T][Hk][d_k]; ``v`` bf16 bits [T][Hv][d_v]
* ``g``, ``beta`` float32 [T][Hv]; ``accept_node`` int32 [B] (-1 = none accepted)

Draw order per workload: tree, acceptance, S0, q, k, v, beta, g, all from one
``numpy.random.default_rng(seed)`` stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Workload", "CONFIGS", "make", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "chain", "root_branch", "random_tree", "accept_by_edge", "tree_depths",
    "zero_pad", "subset", "greedy_tokens", "acceptance_probs",
    "AttnWorkload", "make_attn", "make_attn_small", "make_attn_mixed_b256",
]


# ----------------------------------------------------------------------------
# bf16 helpers (storage format of q, k, v)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    out = ((bits + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# tree shapes
# ----------------------------------------------------------------------------

def chain(n: int) -> np.ndarray:
    """A draft chain of n nodes: node i extends node i-1, node 0 extends S0."""
    return np.arange(-1, n - 1, dtype=np.int32)


def root_branch() -> np.ndarray:
    """Two depth-3 branches hanging off the committed root (6 nodes)."""
    return np.array([-1, 0, 1, -1, 3, 4], dtype=np.int32)


def tree_depths(parent: np.ndarray) -> np.ndarray:
    """Depth of each node, nodes attached to S0 having depth 1."""
    dep = np.zeros(len(parent), dtype=np.int32)
    for i, p in enumerate(parent):
        dep[i] = 1 if p < 0 else dep[p] + 1
    return dep


def random_tree(rng: np.random.Generator, n: int, max_depth: int = 6) -> np.ndarray:
    """Random tree in parent-before-child order with a depth cap.

    parent[i] is uniform over {-1} and the earlier nodes whose depth is below
    the cap, so every node's depth stays <= max_depth.
    """
    parent = np.empty(n, dtype=np.int32)
    dep = np.empty(n, dtype=np.int32)
    for i in range(n):
        eligible = [-1] + [j for j in range(i) if dep[j] < max_depth]
        p = eligible[int(rng.integers(len(eligible)))]
        parent[i] = p
        dep[i] = 1 if p < 0 else dep[p] + 1
    return parent


def accept_by_edge(rng: np.random.Generator, parent: np.ndarray, p_edge: float = 0.7) -> int:
    """Synthetic acceptance: walk down from S0, trying children in index order.

    Each child is accepted independently with probability p_edge; the walk
    enters the first accepted child and stops at a leaf or when every child is
    rejected.  Returns the last accepted node, or -1 when none is.
    """
    children: Dict[int, List[int]] = {}
    for i, p in enumerate(parent):
        children.setdefault(int(p), []).append(i)
    cur = -1
    while True:
        nxt = -1
        for c in children.get(cur, []):
            if rng.random() < p_edge:
                nxt = c
                break
        if nxt < 0:
            return cur
        cur = nxt


# ----------------------------------------------------------------------------
# workload container
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    B: int
    Hv: int
    Hk: int
    d: int
    node_offset: np.ndarray            # int32 [B+1]
    parent: np.ndarray                 # int32 [T]
    accept_node: np.ndarray            # int32 [B]
    S0: np.ndarray                     # float32/float64 [B][Hv][d][d]
    q: np.ndarray                      # bf16 bits [T][Hk][d]  (float64 when fp64)
    k: np.ndarray
    v: np.ndarray                      # bf16 bits [T][Hv][d]  (float64 when fp64)
    g: np.ndarray                      # float32/float64 [T][Hv]
    beta: np.ndarray
    fp64: bool = False
    kinds: Optional[List[str]] = None  # per-request tree kind (mixed batches)
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.node_offset[-1])

    @property
    def max_nodes(self) -> int:
        n = np.diff(self.node_offset)
        return int(n.max()) if len(n) else 0

    def nodes(self, b: int) -> int:
        return int(self.node_offset[b + 1] - self.node_offset[b])

    def parents_of(self, b: int) -> np.ndarray:
        return self.parent[self.node_offset[b]:self.node_offset[b + 1]]

    # values as the device sees them, widened to float64 for the oracle
    def q64(self) -> np.ndarray:
        return self.q.astype(np.float64) if self.fp64 else bf16_bits_to_f32(self.q).astype(np.float64)

    def k64(self) -> np.ndarray:
        return self.k.astype(np.float64) if self.fp64 else bf16_bits_to_f32(self.k).astype(np.float64)

    def v64(self) -> np.ndarray:
        return self.v.astype(np.float64) if self.fp64 else bf16_bits_to_f32(self.v).astype(np.float64)


def _assemble(name, rng, parents, accepts, Hv, Hk, d, s0_var, fp64=False, kinds=None):
    """Draw S0, q, k, v, beta, g (in that order) for an already drawn forest."""
    B = len(parents)
    counts = np.array([len(p) for p in parents], dtype=np.int64)
    node_offset = np.zeros(B + 1, dtype=np.int32)
    node_offset[1:] = np.cumsum(counts)
    T = int(node_offset[-1])
    parent = np.concatenate(parents).astype(np.int32) if T else np.zeros(0, np.int32)
    accept = np.asarray(accepts, dtype=np.int32)
    std = float(np.sqrt(s0_var))
    if fp64:
        S0 = rng.standard_normal((B, Hv, d, d)) * std
        q = rng.standard_normal((T, Hk, d))
        k = rng.standard_normal((T, Hk, d))
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((T, Hv, d))
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))
        g = -np.logaddexp(0.0, rng.standard_normal((T, Hv)))
    else:
        S0 = rng.standard_normal((B, Hv, d, d), dtype=np.float32)
        S0 *= np.float32(std)
        q32 = rng.standard_normal((T, Hk, d), dtype=np.float32)
        k32 = rng.standard_normal((T, Hk, d), dtype=np.float32)
        k32 /= np.linalg.norm(k32, axis=-1, keepdims=True).astype(np.float32)
        v32 = rng.standard_normal((T, Hv, d), dtype=np.float32)
        q, k, v = f32_to_bf16_bits(q32), f32_to_bf16_bits(k32), f32_to_bf16_bits(v32)
        zb = rng.standard_normal((T, Hv), dtype=np.float32)
        beta = (1.0 / (1.0 + np.exp(-zb.astype(np.float64)))).astype(np.float32)
        zg = rng.standard_normal((T, Hv), dtype=np.float32)
        g = (-np.logaddexp(0.0, zg.astype(np.float64))).astype(np.float32)
    return Workload(name=name, B=B, Hv=Hv, Hk=Hk, d=d, node_offset=node_offset, parent=parent,
                    accept_node=accept, S0=S0, q=q, k=k, v=v, g=g, beta=beta, fp64=fp64,
                    kinds=kinds)


# ----------------------------------------------------------------------------
# the five configurations
# ----------------------------------------------------------------------------

def _deepest_first_index(parent: np.ndarray) -> int:
    dep = tree_depths(parent)
    return int(np.argmax(dep))      # ties go to the lowest index


def make_tiny_d16(kind: str = "chain", seed: int = 0) -> Workload:
    """1 request, 1 head, d=16, fp64 inputs; a 4-node chain or the 5-node tree
    [-1,0,0,1,2]; accepted path = root to the deepest node (lowest index on a tie)."""
    rng = np.random.default_rng(seed)
    parent = chain(4) if kind == "chain" else np.array([-1, 0, 0, 1, 2], dtype=np.int32)
    acc = _deepest_first_index(parent)
    return _assemble(f"tiny_d16_{kind}", rng, [parent], [acc], Hv=1, Hk=1, d=16, s0_var=1.0 / 16, fp64=True)


def make_chain3_b64(seed: int = 0, B: int = 64) -> Workload:
    """Depth-3 draft chains, 64 requests x 32 v-heads (16 k-heads), accepted
    length uniform in {0..3}."""
    rng = np.random.default_rng(seed)
    parents = [chain(3) for _ in range(B)]
    accepts = [int(rng.integers(0, 4)) - 1 for _ in range(B)]
    return _assemble("chain3_b64", rng, parents, accepts, Hv=32, Hk=16, d=128, s0_var=0.02)


def make_root_branch6(B: int = 16, seed: int = 0, bfs: bool = False) -> Workload:
    """6-node root-branch trees, batch 1 or 16, 32 v-heads (16 k-heads), S0 with
    variance 1/16; the accepted node is uniform over {none} and the nodes."""
    rng = np.random.default_rng(seed)
    base = np.array([-1, -1, 0, 1, 2, 3], dtype=np.int32) if bfs else root_branch()
    parents = [base.copy() for _ in range(B)]
    accepts = [int(rng.integers(0, 7)) - 1 for _ in range(B)]
    return _assemble(f"rootbranch6_b{B}" + ("_bfs" if bfs else ""), rng, parents, accepts,
                     Hv=32, Hk=16, d=128, s0_var=1.0 / 16)


def make_random32_b256(seed: int = 0, B: int = 256, n: int = 32, Hv: int = 32, Hk: int = 16) -> Workload:
    """Random 32-node trees (depth <= 6), batch 256, 32 v-heads / 16 k-heads,
    acceptance 0.7 per edge."""
    rng = np.random.default_rng(seed)
    parents = [random_tree(rng, n) for _ in range(B)]
    accepts = [accept_by_edge(rng, p) for p in parents]
    return _assemble(f"random{n}_b{B}", rng, parents, accepts, Hv=Hv, Hk=Hk, d=128, s0_var=0.02)


MIXED_KINDS = ("chain3", "rootbranch6", "random16", "random64")


def make_mixed_b256(seed: int = 0, per_kind: int = 64, Hv: int = 48, Hk: int = 16) -> Workload:
    """Ragged batch: per_kind requests of each of chain-3, root-branch-6,
    random-16 and random-64 trees in a seeded shuffle; 48 v-heads / 16 k-heads."""
    rng = np.random.default_rng(seed)
    kinds = [k for k in MIXED_KINDS for _ in range(per_kind)]
    order = rng.permutation(len(kinds))
    kinds = [kinds[i] for i in order]
    parents = []
    for kd in kinds:
        if kd == "chain3":
            parents.append(chain(3))
        elif kd == "rootbranch6":
            parents.append(root_branch())
        elif kd == "random16":
            parents.append(random_tree(rng, 16))
        else:
            parents.append(random_tree(rng, 64))
    accepts = [accept_by_edge(rng, p) for p in parents]
    return _assemble(f"mixed_b{len(kinds)}", rng, parents, accepts, Hv=Hv, Hk=Hk, d=128,
                     s0_var=0.02, kinds=kinds)


def make_custom(parents: List[np.ndarray], accepts: List[int], Hv: int = 4, Hk: int = 2, d: int = 128,
                s0_var: float = 0.02, seed: int = 0, name: str = "custom") -> Workload:
    """Arbitrary forest with the standard value distributions (test helper)."""
    rng = np.random.default_rng(seed)
    return _assemble(name, rng, [np.asarray(p, np.int32) for p in parents], accepts,
                     Hv=Hv, Hk=Hk, d=d, s0_var=s0_var)


CONFIGS = {
    "tiny_d16_chain": lambda: make_tiny_d16("chain"),
    "tiny_d16_tree": lambda: make_tiny_d16("tree"),
    "chain3_b64": make_chain3_b64,
    "rootbranch6_b1": lambda: make_root_branch6(B=1),
    "rootbranch6_b16": lambda: make_root_branch6(B=16),
    "rootbranch6_b16_bfs": lambda: make_root_branch6(B=16, bfs=True),
    "random32_b256": make_random32_b256,
    "mixed_b256": make_mixed_b256,
}


def make(name: str) -> Workload:
    return CONFIGS[name]()


# ----------------------------------------------------------------------------
# reshaping helpers (no arithmetic on values beyond exact rounding/padding)
# ----------------------------------------------------------------------------

def zero_pad(wl: Workload, d: int = 128) -> Workload:
    """Round an fp64 workload to the device formats (bf16 q/k/v, fp32 S0/g/beta)
    and embed it in d dimensions with zeros."""
    d0 = wl.d
    T, B = wl.T, wl.B

    def pad_rows(x, H):
        out = np.zeros((x.shape[0], H, d), dtype=np.float32)
        out[:, :, :d0] = x
        return out

    q = f32_to_bf16_bits(pad_rows(np.asarray(wl.q, np.float32), wl.Hk))
    k = f32_to_bf16_bits(pad_rows(np.asarray(wl.k, np.float32), wl.Hk))
    v = f32_to_bf16_bits(pad_rows(np.asarray(wl.v, np.float32), wl.Hv))
    S0 = np.zeros((B, wl.Hv, d, d), dtype=np.float32)
    S0[:, :, :d0, :d0] = wl.S0
    return Workload(name=wl.name + f"_pad{d}", B=B, Hv=wl.Hv, Hk=wl.Hk, d=d,
                    node_offset=wl.node_offset.copy(), parent=wl.parent.copy(),
                    accept_node=wl.accept_node.copy(), S0=S0, q=q, k=k, v=v,
                    g=np.asarray(wl.g, np.float32), beta=np.asarray(wl.beta, np.float32),
                    fp64=False, kinds=wl.kinds)


def subset(wl: Workload, requests) -> Workload:
    """The workload restricted to the listed requests (in the given order)."""
    reqs = [int(b) for b in requests]
    rows = [np.arange(wl.node_offset[b], wl.node_offset[b + 1]) for b in reqs]
    idx = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    counts = np.array([len(r) for r in rows], dtype=np.int64)
    off = np.zeros(len(reqs) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return Workload(name=wl.name + "_sub", B=len(reqs), Hv=wl.Hv, Hk=wl.Hk, d=wl.d, node_offset=off,
                    parent=wl.parent[idx].copy(), accept_node=wl.accept_node[reqs].copy(),
                    S0=wl.S0[reqs].copy(), q=wl.q[idx].copy(), k=wl.k[idx].copy(),
                    v=wl.v[idx].copy(), g=wl.g[idx].copy(), beta=wl.beta[idx].copy(),
                    fp64=wl.fp64, kinds=[wl.kinds[b] for b in reqs] if wl.kinds else None)


# ----------------------------------------------------------------------------
# token ids for greedy acceptance (synthetic: no model, no vocabulary file)
# ----------------------------------------------------------------------------

def greedy_tokens(wl: Workload, vocab: int = 32000, p_match: float = 0.7, seed: int = 1):
    """Draft token per node and the target's greedy prediction after every node
    and after each request's committed context.

    Siblings get distinct draft tokens (a drafter proposes distinct children).
    At every position the target's prediction equals the draft token of one of
    the position's children with probability p_match (that child chosen
    uniformly), else a token no child carries.
    Returns (draft [T], target_next [T], root_next [B]) as int32.
    """
    rng = np.random.default_rng(seed)
    T, B = wl.T, wl.B
    draft = np.zeros(T, dtype=np.int32)
    target = np.zeros(T, dtype=np.int32)
    root = np.zeros(B, dtype=np.int32)
    for b in range(B):
        lo, hi = int(wl.node_offset[b]), int(wl.node_offset[b + 1])
        par = wl.parent[lo:hi]
        kids = {}
        for i, p in enumerate(par):
            kids.setdefault(int(p), []).append(i)
        for p, ch in kids.items():
            toks = rng.choice(vocab, size=len(ch), replace=False)
            for i, tk in zip(ch, toks):
                draft[lo + i] = tk
        for pos in [-1] + list(range(hi - lo)):
            ch = kids.get(pos, [])
            if ch and rng.random() < p_match:
                want = int(draft[lo + ch[int(rng.integers(len(ch)))]])
            else:
                taken = {int(draft[lo + i]) for i in ch}
                want = int(rng.integers(vocab))
                while want in taken:
                    want = int(rng.integers(vocab))
            if pos < 0:
                root[b] = want
            else:
                target[lo + pos] = want
    return draft, target, root


def acceptance_probs(wl: Workload, first: float = 0.75, last: float = 0.08, positions: int = 7,
                     spread: float = 0.08, seed: int = 2) -> np.ndarray:
    """Per-node acceptance probability estimates (float32 [T]) that fall with
    depth: the mean is `first` at depth 1 and `last` at depth `positions`,
    geometric in between and flat beyond (the DSpark page reports the first of
    seven draft tokens accepted more than 70% of the time and the last less
    than 10%), with N(0, spread^2) noise clipped to [0, 1]."""
    rng = np.random.default_rng(seed)
    p = np.zeros(wl.T, dtype=np.float32)
    ratio = (last / first) ** (1.0 / max(1, positions - 1))
    for b in range(wl.B):
        lo = int(wl.node_offset[b])
        dep = tree_depths(wl.parents_of(b))
        mean = first * ratio ** (np.minimum(dep, positions) - 1)
        p[lo:lo + len(dep)] = np.clip(mean + spread * rng.standard_normal(len(dep)), 0.0, 1.0)
    return p


# ----------------------------------------------------------------------------
# Tree-bias attention inputs (the hybrid's attention layers over the same trees)
# ----------------------------------------------------------------------------

@dataclass
class AttnWorkload:
    """Inputs of ancestry-masked decode attention for a draft forest.

    q bf16 bits [T][Hq][d]; k_ctx, v_ctx bf16 bits [C][Hkv][d] (request b's
    committed context is rows ctx_offset[b] .. ctx_offset[b+1]-1);
    k_node, v_node bf16 bits [T][Hkv][d] (the draft nodes' own keys/values);
    node_offset, ctx_offset int32 [B+1]; parent int32 [T]."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    node_offset: np.ndarray
    parent: np.ndarray
    ctx_offset: np.ndarray
    q: np.ndarray
    k_ctx: np.ndarray
    v_ctx: np.ndarray
    k_node: np.ndarray
    v_node: np.ndarray
    scale: float
    kinds: Optional[List[str]] = None

    @property
    def T(self) -> int:
        return int(self.node_offset[-1])

    @property
    def C(self) -> int:
        return int(self.ctx_offset[-1])

    @property
    def max_nodes(self) -> int:
        return int(np.max(np.diff(self.node_offset))) if self.B else 1

    @property
    def max_ctx(self) -> int:
        return int(np.max(np.diff(self.ctx_offset))) if self.B else 0

    def f32(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, name))


def _bf16_normal(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0, 1) draws rounded to bf16 bits (nearest even), produced in chunks so
    that multi-GB arrays need no float64 or uint64 temporaries."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        bits = rng.standard_normal(m, dtype=np.float32).view(np.uint32)
        out[i:i + m] = ((bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    return out.reshape(shape)


CTX_POOL = 32768


def make_attn(parents: List[np.ndarray], ctx_lens: List[int], Hq: int = 32, Hkv: int = 8, d: int = 128,
              seed: int = 0, name: str = "attn", kinds=None) -> AttnWorkload:
    """q, k, v ~ N(0, 1) rounded to bf16; context keys/values are rows of a pool
    of min(C, CTX_POOL) such rows per array (all of them, in order, when C fits;
    else drawn with replacement); scale 1/sqrt(d).  Draw order: q, k_node,
    v_node, pool row choice, k pool, v pool."""
    rng = np.random.default_rng(seed)
    sizes = [len(p) for p in parents]
    node_offset = np.zeros(len(parents) + 1, dtype=np.int32)
    node_offset[1:] = np.cumsum(sizes)
    ctx_offset = np.zeros(len(parents) + 1, dtype=np.int32)
    ctx_offset[1:] = np.cumsum(ctx_lens)
    T, C = int(node_offset[-1]), int(ctx_offset[-1])
    parent = np.concatenate([np.asarray(p, dtype=np.int32) for p in parents]) if T else np.zeros(0, np.int32)
    bf = lambda shape: _bf16_normal(rng, shape)
    q = bf((T, Hq, d))
    k_node = bf((T, Hkv, d))
    v_node = bf((T, Hkv, d))
    # context rows: up to CTX_POOL distinct rows; longer caches reuse pool rows
    # drawn with replacement (drawing every row of a multi-GB cache is too slow)
    P = min(C, CTX_POOL)
    idx = np.arange(C) if C <= P else rng.integers(0, P, size=C)
    k_ctx = bf((P, Hkv, d))[idx]
    v_ctx = bf((P, Hkv, d))[idx]
    return AttnWorkload(name, len(parents), Hq, Hkv, d, node_offset, parent, ctx_offset, q, k_ctx, v_ctx,
                        k_node, v_node, 1.0 / float(np.sqrt(d)), kinds)


def make_attn_small(seed: int = 0) -> AttnWorkload:
    """Edge mix for parity: empty context, one key, block-boundary lengths, a
    forest, a 64-node tree, an empty request; 8 query heads over 2 kv heads."""
    rng = np.random.default_rng(seed + 100)
    parents = [chain(3), root_branch(), np.array([-1, -1, 0], np.int32), np.array([-1], np.int32),
               random_tree(rng, 16), random_tree(rng, 64), np.zeros(0, np.int32), chain(5)]
    ctx = [0, 1, 63, 64, 65, 200, 7, 130]
    return make_attn(parents, ctx, Hq=8, Hkv=2, seed=seed, name="attn_small")


def make_attn_mixed_b256(seed: int = 0, ctx_lo: int = 1024, ctx_hi: int = 4096, Hq: int = 32, Hkv: int = 8) -> AttnWorkload:
    """The mixed batch-256 trees (64 each of chain-3, root-branch-6, random-16,
    random-64, shuffled) with committed contexts uniform in [ctx_lo, ctx_hi]."""
    wl = make_mixed_b256(seed)
    parents = [wl.parents_of(b) for b in range(wl.B)]
    rng = np.random.default_rng(seed + 7)
    ctx = [int(x) for x in rng.integers(ctx_lo, ctx_hi + 1, size=wl.B)]
    return make_attn(parents, ctx, Hq=Hq, Hkv=Hkv, seed=seed + 11, name="attn_mixed_b256", kinds=wl.kinds)
