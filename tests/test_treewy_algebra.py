"""The tree-structured WY form of the gated delta rule, in fp64, against the oracle.

TreeWY (abstract, "Method", "Novelty") computes all pseudo-values of a draft
tree with one triangular system whose off-diagonal entries only couple a node
with its ancestors (parent-before-child order makes it lower triangular),
reads every node's output from those pseudo-values, and rebuilds the accepted
state from the accepted path's pseudo-values alone.  The identities written
out below are derived from the sequential rule:

  G_t = sum of g over the inclusive ancestors of t;  gamma_t = exp(G_t)
  D_tj = exp(G_t - G_j) for j an inclusive ancestor of t, else 0
  S_t  = gamma_t S0 + sum_{j in anc*(t)} D_tj u_j k_j^T                      (A1)
  u_t + beta_t sum_{j in anc(t)} D_tj (k_t.k_j) u_j = beta_t (v_t - gamma_t S0 k_t)  (A2)
  o_t  = gamma_t S0 q_t + sum_{j in anc*(t)} D_tj (q_t.k_j) u_j              (A3)
  S'   = S_a for the accepted node a                                          (A4)

This file is an independent implementation (a dense masked system solved with
scipy's triangular solver); it shares nothing with the oracle except the
inputs.  Agreement to ~1e-12 both pins the oracle from a second formulation
and checks the identities that the HIP kernels implement.
"""
import itertools

import numpy as np
import pytest
from scipy.linalg import solve_triangular

import oracle as O


def treewy_unit(H0, q, k, v, g, beta, parent):
    N = len(parent)
    S0 = H0.T
    M = np.zeros((N, N), dtype=bool)              # inclusive ancestor mask
    for t in range(N):
        j = t
        while j >= 0:
            M[t, j] = True
            j = parent[j]
    G = M.astype(float) @ g                          # path-cumulative log decay
    gam = np.exp(G)
    D = np.where(M, np.exp(np.subtract.outer(G, G)), 0.0)
    Mstrict = M & ~np.eye(N, dtype=bool)
    A = beta[:, None] * np.where(Mstrict, D * (k @ k.T), 0.0)
    R = beta[:, None] * (v - gam[:, None] * (k @ S0.T))
    U = solve_triangular(np.eye(N) + A, R, lower=True, unit_diagonal=True)
    Ot = gam[:, None] * (q @ S0.T) + np.where(M, D * (q @ k.T), 0.0) @ U
    states = [gam[t] * S0 + (D[t][:, None] * U).T @ k for t in range(N)]
    return Ot, U, states


def _inputs(rng, n, d):
    H0 = rng.standard_normal((d, d)) * 0.2
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, d))
    g = -np.logaddexp(0, rng.standard_normal(n))
    beta = 1 / (1 + np.exp(-rng.standard_normal(n)))
    return H0, q, k, v, g, beta


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_all_small_trees(n):
    rng = np.random.default_rng(100 + n)
    H0, q, k, v, g, beta = _inputs(rng, n, 6)
    for par in itertools.product(*[range(-1, i) for i in range(n)]):
        O1, U1, S1 = O.verify_unit(H0, q, k, v, g, beta, par)
        O2, U2, S2 = treewy_unit(H0, q, k, v, g, beta, list(par))
        np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(U2, U1, rtol=1e-12, atol=1e-12)
        for t in range(n):
            np.testing.assert_allclose(S2[t], S1[t], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_random_64_node_trees_d128(seed):
    import workloads as W
    rng = np.random.default_rng(seed)
    par = W.random_tree(rng, 64)
    H0, q, k, v, g, beta = _inputs(rng, 64, 128)
    O1, U1, S1 = O.verify_unit(H0, q, k, v, g, beta, par)
    O2, U2, S2 = treewy_unit(H0, q, k, v, g, beta, list(par))
    scale = np.abs(O1).max()
    assert np.abs(O2 - O1).max() <= 1e-11 * scale
    assert np.abs(U2 - U1).max() <= 1e-11 * np.abs(U1).max()
    a = int(np.argmax(W.tree_depths(par)))
    assert np.abs(S2[a] - S1[a]).max() <= 1e-11 * np.abs(S1[a]).max()
