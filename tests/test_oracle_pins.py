"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each check is chosen so that a plausible mistake in the oracle (a dropped
term, a wrong sign, a transposed outer product, a wrong parent index, a branch
that reads its sibling) fails at least one of them:

* gated_delta_step: the delta rule is one gradient step of size beta on the
  least-squares loss 1/2 ||X k - v||^2 taken at the decayed state X = alpha S;
  the gradient is measured by central finite differences of the loss (exact for
  a quadratic up to rounding), not by the oracle's formula.  Plus the rule's
  defining write property, the untouched orthogonal complement and the
  alpha = 0 / beta = 0 closed forms, and the storage-layout definition.
* verify_unit: brute-force replay of every root-to-node path of every tree up
  to 6 nodes (GDN Tree-Scan: each node must see native sequential decode along
  its root-to-node path), sibling invariance (TreeWY, Method), relabelling.
* commit: equals the accepted node's state; empty path keeps S0; composition.
* storeall: the pages' state count for a depth-3 chain.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd_unit(rng, d, Hk=None):
    x = rng.standard_normal(d)
    return x / np.linalg.norm(x)


# ----------------------------------------------------------------------------
# the single step
# ----------------------------------------------------------------------------

def _loss(X, k, v):
    r = X @ k - v
    return 0.5 * float(r @ r)


@pytest.mark.parametrize("seed", range(5))
def test_step_is_gradient_step_on_least_squares(seed):
    rng = np.random.default_rng(seed)
    dv, dk = 5, 4                                  # non-square: catches transposes
    S = rng.standard_normal((dv, dk))
    k, v, q = rng.standard_normal(dk), rng.standard_normal(dv), rng.standard_normal(dk)
    g, beta = -abs(rng.standard_normal()), 1 / (1 + math.exp(-rng.standard_normal()))
    alpha = math.exp(g)
    X = alpha * S
    grad = np.zeros_like(X)
    h = 1e-3
    for i in range(dv):
        for j in range(dk):
            E = np.zeros_like(X)
            E[i, j] = h
            grad[i, j] = (_loss(X + E, k, v) - _loss(X - E, k, v)) / (2 * h)
    S_new, u, o = O.gated_delta_step(S, q, k, v, g, beta)
    np.testing.assert_allclose(S_new, X - beta * grad, rtol=0, atol=1e-9)
    # the pseudo-value is minus beta times the residual of the decayed state
    np.testing.assert_allclose(u, -beta * (X @ k - v), rtol=0, atol=1e-12)
    # the output is the updated state applied to the query
    np.testing.assert_allclose(o, S_new @ q, rtol=0, atol=1e-12)


@pytest.mark.parametrize("g", [0.0, -0.3, -4.0])
def test_step_writes_association_exactly_when_beta_is_one(g):
    rng = np.random.default_rng(1)
    d = 8
    S = rng.standard_normal((d, d))
    k = rnd_unit(rng, d)
    v = rng.standard_normal(d)
    S_new, _, o = O.gated_delta_step(S, k, k, v, g, 1.0)
    np.testing.assert_allclose(S_new @ k, v, atol=1e-12)
    np.testing.assert_allclose(o, v, atol=1e-12)


def test_step_partial_write_and_orthogonal_complement():
    rng = np.random.default_rng(2)
    d = 7
    S = rng.standard_normal((d, d))
    k = rnd_unit(rng, d)
    v, q = rng.standard_normal(d), rng.standard_normal(d)
    g, beta = -0.7, 0.35
    alpha = math.exp(g)
    S_new, _, _ = O.gated_delta_step(S, q, k, v, g, beta)
    # prediction error along k shrinks by (1 - beta)
    np.testing.assert_allclose(S_new @ k - v, (1 - beta) * (alpha * S @ k - v), atol=1e-12)
    # directions orthogonal to k are only decayed
    x = rng.standard_normal(d)
    x -= (x @ k) * k
    np.testing.assert_allclose(S_new @ x, alpha * (S @ x), atol=1e-12)


def test_step_closed_forms():
    rng = np.random.default_rng(3)
    d = 6
    S = rng.standard_normal((d, d))
    k, v, q = rnd_unit(rng, d), rng.standard_normal(d), rng.standard_normal(d)
    # alpha = 0: the old state is forgotten entirely
    S_new, u, o = O.gated_delta_step(S, q, k, v, -1e4, 0.6)
    np.testing.assert_allclose(S_new, 0.6 * np.outer(v, k), atol=1e-14)
    np.testing.assert_allclose(o, 0.6 * (k @ q) * v, atol=1e-14)
    # beta = 0: pure decay, zero pseudo-value
    S_new, u, o = O.gated_delta_step(S, q, k, v, -0.25, 0.0)
    assert np.all(u == 0)
    np.testing.assert_allclose(S_new, math.exp(-0.25) * S, atol=1e-15)


def test_scalar_case_by_hand():
    # d = 1: s' = alpha*s*(1 - beta*k^2) + beta*v*k.  s=0.5, k=1, v=2,
    # beta=0.5, alpha=0.5: s' = 0.5*0.5*0.5 + 0.5*2 = 1.125; o = s'*q with q = 2.
    S_new, u, o = O.gated_delta_step(np.array([[0.5]]), np.array([2.0]), np.array([1.0]),
                                     np.array([2.0]), math.log(0.5), 0.5)
    assert abs(S_new[0, 0] - 1.125) < 1e-15
    assert abs(u[0] - 0.875) < 1e-15           # 0.5 * (2 - 0.5*0.5*1)
    assert abs(o[0] - 2.25) < 1e-15


def test_storage_layout_row_is_value_of_basis_key():
    """H0 is stored [d_k][d_v]: with beta = 0 and no decay, querying e_i returns row i."""
    rng = np.random.default_rng(4)
    dk = dv = 5
    H0 = rng.standard_normal((dk, dv))
    N = dk
    q = np.eye(dk)
    k = np.tile(rnd_unit(rng, dk), (N, 1))
    v = rng.standard_normal((N, dv))
    Ot, Ut, _ = O.verify_unit(H0, q, k, v, np.zeros(N), np.zeros(N), [-1] * N)
    np.testing.assert_array_equal(Ot, H0)
    assert np.all(Ut == 0)


# ----------------------------------------------------------------------------
# tree structure and path semantics
# ----------------------------------------------------------------------------

def all_trees(n):
    """Every parent array of n nodes in parent-before-child order."""
    return itertools.product(*[range(-1, i) for i in range(n)])


def brute_ancestors(parent, t):
    s = set()
    while t >= 0:
        s.add(t)
        t = parent[t]
    return s


@pytest.mark.parametrize("n", range(1, 7))
def test_ancestry_and_depths_by_brute_force(n):
    for par in all_trees(n):
        anc = O.ancestry(par)
        dep = O.depths(par)
        for t in range(n):
            s = brute_ancestors(par, t)
            assert anc[t] == sum(1 << j for j in s)
            assert dep[t] == len(s) == bin(anc[t]).count("1")


def test_chain_ancestry_closed_form():
    par = list(range(-1, 63))
    anc = O.ancestry(par)
    assert all(anc[t] == (1 << (t + 1)) - 1 for t in range(64))


def test_pages_branch_example_and_root_branch():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    ex = facts["two_branch_reference"]
    anc = O.ancestry(ex["parent"])
    for t, want in enumerate(ex["inclusive_ancestors"]):
        assert anc[t] == sum(1 << j for j in want)
    rb = facts["root_branch_tree"]
    assert O.depths(rb["parent"]) == rb["depths"]


def test_accepted_path_structure():
    rng = np.random.default_rng(5)
    for n in (1, 5, 32, 64):
        for _ in range(20):
            par = [int(rng.integers(-1, i)) if i else -1 for i in range(n)]
            a = int(rng.integers(-1, n))
            p = O.accepted_path(par, a)
            if a < 0:
                assert p == []
                continue
            assert p[-1] == a and par[p[0]] == -1
            assert all(par[p[i]] == p[i - 1] for i in range(1, len(p)))
            assert len(p) == O.depths(par)[a]


def _unit_inputs(rng, n, d, dv=None):
    dv = dv or d
    H0 = rng.standard_normal((d, dv)) * 0.3
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv))
    g = -np.logaddexp(0, rng.standard_normal(n))
    beta = 1 / (1 + np.exp(-rng.standard_normal(n)))
    return H0, q, k, v, g, beta


@pytest.mark.parametrize("n", range(1, 7))
def test_every_node_equals_root_to_node_replay(n):
    """GDN Tree-Scan: a node must carry the state of native sequential decode
    along its root-to-node path.  Replayed from a fresh S0 for every node of
    every tree of n nodes; must be bit-identical to the tree walk."""
    rng = np.random.default_rng(10 + n)
    d, dv = 3, 2
    H0, q, k, v, g, beta = _unit_inputs(rng, n, d, dv)
    for par in all_trees(n):
        Ot, Ut, states = O.verify_unit(H0, q, k, v, g, beta, par)
        for t in range(n):
            S = H0.T.copy()
            for j in O.root_to_node(par, t):
                S, u, o = O.gated_delta_step(S, q[j], k[j], v[j], g[j], beta[j])
            assert np.array_equal(S, states[t])
            assert np.array_equal(u, Ut[t])
            assert np.array_equal(o, Ot[t])


def test_chain_equals_plain_sequential_decode():
    rng = np.random.default_rng(6)
    n, d = 9, 4
    H0, q, k, v, g, beta = _unit_inputs(rng, n, d)
    Ot, Ut, states = O.verify_unit(H0, q, k, v, g, beta, list(range(-1, n - 1)))
    S = H0.T.copy()
    for t in range(n):
        S, u, o = O.gated_delta_step(S, q[t], k[t], v[t], g[t], beta[t])
        assert np.array_equal(o, Ot[t]) and np.array_equal(S, states[t])


def subtree(par, j):
    return {t for t in range(len(par)) if j in brute_ancestors(par, t)}


@pytest.mark.parametrize("seed", range(4))
def test_sibling_invariance(seed):
    """TreeWY, Method: a branch refers to its ancestors only, never another
    branch.  Perturbing node j changes nothing outside subtree(j)."""
    rng = np.random.default_rng(seed)
    n, d = 12, 4
    par = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
    H0, q, k, v, g, beta = _unit_inputs(rng, n, d)
    O0, U0, _ = O.verify_unit(H0, q, k, v, g, beta, par)
    for j in range(n):
        q2, k2, v2, g2, b2 = q.copy(), k.copy(), v.copy(), g.copy(), beta.copy()
        q2[j] += 1.0
        k2[j] = -k2[j]
        v2[j] *= 3.0
        g2[j] -= 0.5
        b2[j] = 0.9
        O1, U1, _ = O.verify_unit(H0, q2, k2, v2, g2, b2, par)
        inside = subtree(par, j)
        for t in range(n):
            if t not in inside:
                assert np.array_equal(O0[t], O1[t]) and np.array_equal(U0[t], U1[t])
            else:
                assert not np.array_equal(O0[t], O1[t])


@pytest.mark.parametrize("kind", ["nan_g", "nan_beta", "inf_v"])
def test_non_finite_input_stays_in_its_subtree(kind):
    """TreeWY, Method: a branch reads only its common ancestors, never the other
    branch, so a NaN or Inf in one node's inputs reaches its subtree and nothing
    else: every other node's output and pseudo-value keep their bits.  Inside the
    subtree it reaches exactly the value rows it touches: under the gated delta
    rule row i of the state is updated from component i of v and of u alone
    (u_i = beta (v_i - alpha (S k)_i), S_i. <- alpha S_i. + u_i k^T), so an Inf in
    v[c] makes column c non-finite in the subtree and leaves the other columns'
    bits unchanged, while a NaN gate or beta spoils every column there."""
    rng = np.random.default_rng(21)
    n, d = 14, 6
    par = [-1, 0, 1, 0, 3, 4, -1, 6, 2, 8, 5, 3, 11, 7]
    H0, q, k, v, g, beta = _unit_inputs(rng, n, d)
    O0, U0, _ = O.verify_unit(H0, q, k, v, g, beta, par)
    for j in (1, 3, 6):
        g2, b2, v2 = g.copy(), beta.copy(), v.copy()
        if kind == "nan_g":
            g2[j] = np.nan
        elif kind == "nan_beta":
            b2[j] = np.nan
        else:
            v2[j, 2] = np.inf
        with np.errstate(invalid="ignore", over="ignore"):
            O1, U1, _ = O.verify_unit(H0, q, k, v2, g2, b2, par)
        inside = subtree(par, j)
        for t in range(n):
            if t not in inside:
                assert np.array_equal(O0[t], O1[t]) and np.array_equal(U0[t], U1[t]), (j, t)
            elif kind == "inf_v":
                other = [c for c in range(d) if c != 2]
                assert not np.isfinite(O1[t, 2]) and not np.isfinite(U1[t, 2]), (j, t)
                assert np.array_equal(O0[t, other], O1[t, other]) and np.array_equal(U0[t, other], U1[t, other])
            else:
                assert not np.isfinite(O1[t]).any() and not np.isfinite(U1[t]).any(), (j, t)


def test_relabelling_permutes_results():
    """Another parent-before-child order of the same tree permutes the outputs."""
    rng = np.random.default_rng(7)
    # tree: 0 root; 1,2 children of 0; 3 child of 1; 4 child of 2; 5 root
    par = [-1, 0, 0, 1, 2, -1]
    # BFS-like relabelling: new order of old nodes
    order = [5, 0, 2, 1, 4, 3]
    newidx = {old: i for i, old in enumerate(order)}
    par2 = [-1 if par[o] < 0 else newidx[par[o]] for o in order]
    assert O.parents_valid(par2)
    n, d = 6, 4
    H0, q, k, v, g, beta = _unit_inputs(rng, n, d)
    O1, U1, _ = O.verify_unit(H0, q, k, v, g, beta, par)
    O2, U2, _ = O.verify_unit(H0, q[order], k[order], v[order], g[order], beta[order], par2)
    assert np.array_equal(O1[order], O2) and np.array_equal(U1[order], U2)


# ----------------------------------------------------------------------------
# commit
# ----------------------------------------------------------------------------

def test_commit_equals_accepted_state_and_empty_keeps_S0():
    rng = np.random.default_rng(8)
    n, d = 10, 4
    par = [-1, 0, 1, 0, 3, -1, 5, 6, 2, 8]
    H0, q, k, v, g, beta = _unit_inputs(rng, n, d)
    _, _, states = O.verify_unit(H0, q, k, v, g, beta, par)
    for a in range(-1, n):
        p = O.accepted_path(par, a)
        c1 = O.commit_unit(H0, states, p)
        c2 = O.replay_commit_unit(H0, q, k, v, g, beta, p)
        assert np.array_equal(c1, c2)
        if a < 0:
            assert np.array_equal(c1, H0)
        else:
            assert np.array_equal(c1, states[a].T)


def test_verify_commit_composition():
    """Verifying a depth-(a+b) chain at once equals verify a, commit, verify b."""
    rng = np.random.default_rng(9)
    a, b, d = 3, 4, 5
    n = a + b
    H0, q, k, v, g, beta = _unit_inputs(rng, n, d)
    Oall, _, states = O.verify_unit(H0, q, k, v, g, beta, list(range(-1, n - 1)))
    O1, _, st1 = O.verify_unit(H0, q[:a], k[:a], v[:a], g[:a], beta[:a], list(range(-1, a - 1)))
    H1 = O.commit_unit(H0, st1, list(range(a)))
    O2, _, st2 = O.verify_unit(H1, q[a:], k[a:], v[a:], g[a:], beta[a:], list(range(-1, b - 1)))
    np.testing.assert_allclose(np.concatenate([O1, O2]), Oall, rtol=0, atol=1e-13)
    np.testing.assert_allclose(st2[-1], states[-1], rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------
# storeall and memory accounting
# ----------------------------------------------------------------------------

def test_storeall_state_count_matches_pages():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    want = facts["storeall_state_count_depth3_chain"]["value"]
    d = 128
    per_state = d * d * 4
    spec = O.state_bytes(1, 1, d, d, 3, storeall=True) // per_state
    assert spec + 1 == want          # plus the committed state itself
    # the tree-WY path keeps no extra state, only U rows
    assert O.state_bytes(1, 1, d, d, 3, storeall=False) == 3 * d * 4


def test_storeall_batch_states_are_path_states():
    import workloads as W
    wl = W.make_custom([W.chain(3), W.root_branch()], [1, 4], Hv=2, Hk=1, d=8, seed=3)
    args = (wl.S0, wl.q64(), wl.k64(), wl.v64(), wl.g, wl.beta, wl.node_offset, wl.parent, wl.Hv, wl.Hk)
    Ob, NS, st = O.verify_storeall_batch(*args)
    assert np.all(st == 0)
    for b in range(wl.B):
        lo = wl.node_offset[b]
        par = wl.parents_of(b)
        for h in range(wl.Hv):
            for t in range(wl.nodes(b)):
                p = O.root_to_node(par, t)
                want = O.replay_commit_unit(wl.S0[b, h].astype(np.float64), wl.q64()[lo:, h // 2],
                                            wl.k64()[lo:, h // 2], wl.v64()[lo:, h],
                                            wl.g[lo:, h].astype(np.float64),
                                            wl.beta[lo:, h].astype(np.float64), p)
                assert np.array_equal(NS[lo + t, h], want)
    out, st2 = O.commit_storeall_batch(wl.S0, NS, wl.node_offset, wl.parent, wl.accept_node)
    assert np.array_equal(out[0], NS[1]) and np.array_equal(out[1], NS[3 + 4])


# ----------------------------------------------------------------------------
# error statuses
# ----------------------------------------------------------------------------

def test_statuses():
    import workloads as W
    wl = W.make_custom([W.chain(3), W.chain(2)], [0, 1], Hv=2, Hk=2, d=4)
    par = wl.parent.copy()
    par[4] = 1                                   # request 1, node 1 -> parent 1 (not < 1)
    O_, U_, anc, st = O.verify_batch(wl.S0, wl.q64(), wl.k64(), wl.v64(), wl.g, wl.beta,
                                     wl.node_offset, par, wl.Hv, wl.Hk)
    assert list(st) == [O.STATUS_OK, O.STATUS_BAD_PARENT]
    assert np.isnan(O_[3:]).all() and not np.isnan(O_[:3]).any() and anc[3] == 0
    path = np.zeros((2, 3), np.int32)
    path[0, :2] = [0, 2]                          # 2's parent is 1, not 0
    _, cst = O.commit_batch(wl.S0, wl.q64(), wl.k64(), wl.v64(), wl.g, wl.beta, wl.node_offset,
                            wl.parent, path, np.array([2, 0]), wl.Hv, wl.Hk, max_nodes=3)
    assert list(cst) == [O.STATUS_BAD_PATH, O.STATUS_OK]
    p, pl, pst = O.accepted_path_batch(wl.node_offset, wl.parent, np.array([3, -1]), max_nodes=3)
    assert list(pst) == [O.STATUS_BAD_ACCEPT, O.STATUS_OK] and pl[1] == 0
    off = np.array([0, 3, 2], np.int32)
    _, _, _, st = O.verify_batch(wl.S0, wl.q64(), wl.k64(), wl.v64(), wl.g, wl.beta, off,
                                 wl.parent, wl.Hv, wl.Hk)
    assert st[1] == O.STATUS_BAD_OFFSETS


def test_c1_worked_cases():
    """The small fp64 configuration: 4-node chain and the 5-node tree."""
    import workloads as W
    for kind, want_path in (("chain", [0, 1, 2, 3]), ("tree", [0, 1, 3])):
        wl = W.make_tiny_d16(kind)
        p = O.accepted_path(wl.parent, int(wl.accept_node[0]))
        assert p == want_path
        st, Ob, Ub, anc, states = O.verify_request(wl.S0, wl.q, wl.k, wl.v, wl.g, wl.beta,
                                                   wl.node_offset, wl.parent, 0, 1, 1)
        assert st == 0 and np.all(np.isfinite(Ob))
        H1 = O.commit_unit(wl.S0[0, 0], states[0], p)
        assert np.array_equal(H1, states[0][p[-1]].T)


# ----------------------------------------------------------------------------
# greedy acceptance
# ----------------------------------------------------------------------------

def _all_root_paths(par):
    n = len(par)
    return [O.root_to_node(par, t) for t in range(n)]


@pytest.mark.parametrize("n", range(1, 7))
def test_greedy_accept_is_longest_matching_path(n):
    """With distinct sibling tokens, greedy acceptance equals the longest root-first
    path on which every node's token is the target's prediction at its parent
    (brute force over all paths), for every tree of n nodes."""
    rng = np.random.default_rng(20 + n)
    for par in all_trees(n):
        par = list(par)
        draft = np.zeros(n, dtype=np.int64)
        kids = {}
        for t, p in enumerate(par):
            kids.setdefault(p, []).append(t)
        for p, ch in kids.items():
            draft[ch] = rng.choice(6, size=len(ch), replace=False)
        for _ in range(4):
            tgt = rng.integers(0, 6, size=n)
            root = int(rng.integers(0, 6))
            a = O.greedy_accept(par, draft, tgt, root)
            def ok(path):
                want = root
                for t in path:
                    if draft[t] != want:
                        return False
                    want = tgt[t]
                return True
            best = [p for p in _all_root_paths(par) if ok(p)]
            longest = max((len(p) for p in best), default=0)
            assert len(O.accepted_path(par, a)) == longest
            if a >= 0:
                assert ok(O.root_to_node(par, a))


def test_greedy_accept_chain_prefix():
    par = list(range(-1, 7))
    draft = np.arange(10, 18)
    tgt = np.arange(11, 19).copy()
    assert O.greedy_accept(par, draft, tgt, 10) == 7          # everything matches
    tgt[3] = 0                                                # node 4 no longer predicted
    assert O.greedy_accept(par, draft, tgt, 10) == 3
    assert O.greedy_accept(par, draft, tgt, 99) == -1          # first token already wrong


def test_greedy_tokens_generator_contract():
    import workloads as W
    wl = W.make_mixed_b256(per_kind=4, Hv=2, Hk=1)
    draft, tgt, root = W.greedy_tokens(wl)
    for b in range(wl.B):
        lo = wl.node_offset[b]
        par = wl.parents_of(b)
        kids = {}
        for t, p in enumerate(par):
            kids.setdefault(int(p), []).append(int(draft[lo + t]))
        assert all(len(v) == len(set(v)) for v in kids.values())


# ----------------------------------------------------------------------------
# survival and the load-adaptive budget
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n", range(1, 7))
def test_survival_is_path_product(n):
    rng = np.random.default_rng(30 + n)
    for par in all_trees(n):
        p = rng.random(n).astype(np.float32)
        s = O.survival(par, p)
        for t in range(n):
            want = np.float32(1.0)
            for j in O.root_to_node(par, t):
                want = np.float32(want * p[j]) if j != O.root_to_node(par, t)[0] else p[j]
            assert s[t] == want


def test_survival_chain_closed_form():
    p = np.full(10, 0.5, np.float32)
    s = O.survival(list(range(-1, 9)), p)
    assert np.array_equal(s, (0.5 ** np.arange(1, 11)).astype(np.float32))


@pytest.mark.parametrize("seed", range(4))
def test_budget_select_properties(seed):
    import workloads as W
    wl = W.make_mixed_b256(per_kind=3, Hv=2, Hk=1, seed=seed)
    p = W.acceptance_probs(wl, seed=seed)
    p[::7] = 1.0                                     # exact ties along paths
    for budget, thr in ((0, 0.0), (10, 0.0), (wl.T // 2, 0.05), (wl.T + 5, 0.2), (wl.T, 0.0)):
        s, keep, cnt, st = O.budget_select(wl.node_offset, wl.parent, p, budget, thr)
        assert np.all(st == 0)
        eligible = int((s >= np.float32(thr)).sum())
        # the threshold only removes a suffix of the order, so the count is exact
        assert keep.sum() == min(budget, eligible)
        kept, dropped = s[keep == 1], s[(keep == 0) & (s >= np.float32(thr))]
        if len(kept) and len(dropped):
            assert kept.min() >= dropped.max()
        assert np.all(kept >= np.float32(thr))
        for b in range(wl.B):
            lo = wl.node_offset[b]
            par = wl.parents_of(b)
            for t in range(len(par)):
                if keep[lo + t] and par[t] >= 0:
                    assert keep[lo + par[t]]             # ancestor-closed
            assert cnt[b] == keep[lo:lo + len(par)].sum()


def test_acceptance_probs_follow_pages_decay():
    import workloads as W
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))["dspark_acceptance_by_position"]
    wl = W.make_custom([W.chain(7)] * 400, [0] * 400, Hv=1, Hk=1, d=4)
    p = W.acceptance_probs(wl).reshape(400, 7)
    assert p[:, 0].mean() > facts["first_above"] and p[:, -1].mean() < facts["last_below"]


# ----------------------------------------------------------------------------
# the budget selection's tie order, by hand-built cases
# ----------------------------------------------------------------------------

def _budget_cases():
    return json.load(open(os.path.join(GOLDEN, "budget_ties.json")))["cases"]


def _keep_by_order(case, key):
    """The kept set when the valid nodes are ranked by `key(survival, depth, global index)`:
    a deliberately different ordering, to show that the hand-built cases tell orders apart."""
    off, par, p = case["node_offset"], case["parent"], np.asarray(case["p"], np.float32)
    nodes = []
    for b in range(len(off) - 1):
        lo, hi = off[b], off[b + 1]
        s = O.survival(par[lo:hi], p[lo:hi])
        d = O.depths(par[lo:hi])
        nodes += [(float(s[t]), d[t], lo + t) for t in range(hi - lo)]
    keep = [0] * len(par)
    for s, _, gi in sorted(nodes, key=lambda x: key(*x))[:case["budget"]]:
        if s >= np.float32(case["threshold"]):
            keep[gi] = 1
    return keep


@pytest.mark.parametrize("case", _budget_cases(), ids=lambda c: c["name"])
def test_budget_select_tie_order_hand_cases(case):
    off = np.asarray(case["node_offset"], np.int32)
    par = np.asarray(case["parent"], np.int32)
    p = np.asarray(case["p"], np.float32)
    s, keep, kept, st = O.budget_select(off, par, p, case["budget"], case["threshold"])
    assert np.all(st == 0)
    assert keep.tolist() == case["expected_keep"], case["why"]
    assert kept.tolist() == case["expected_kept"]


def test_budget_tie_cases_reject_other_orders():
    """Every swapped tie-break loses at least one hand-built case: the cases pin the order."""
    cases = _budget_cases()
    assert all(_keep_by_order(c, lambda s, d, i: (-s, d, i)) == c["expected_keep"] for c in cases)
    mutants = {
        "index descending": lambda s, d, i: (-s, d, -i),
        "depth descending": lambda s, d, i: (-s, -d, i),
        "index before depth": lambda s, d, i: (-s, i, d),
        "index only after survival, reversed": lambda s, d, i: (-s, -i),
    }
    for name, key in mutants.items():
        assert any(_keep_by_order(c, key) != c["expected_keep"] for c in cases), name
