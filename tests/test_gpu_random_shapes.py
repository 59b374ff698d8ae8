"""Seeded random shapes through the two-launch and the one-launch decoding step.

Batch sizes, key-head counts (including ones that are not multiples of 8 or 16,
which take other workgroup deals), grouped-query ratios, trees from empty to 64
nodes (random trees and chains), random accepted nodes.  Each case: the
one-launch commit + verify equals commit_node followed by verify bit for bit
(states, outputs, pseudo-values, masks, statuses), and both match the oracle's
commit-then-verify.
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity_commit_verify import assert_same_bits, oracle_check, run_pair

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 2, 3, 5, 6, 15, 16, 17, 31, 32, 33, 48, 63, 64]


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    Hk = int(rng.choice([1, 2, 3, 5, 8, 16]))
    r = int(rng.choice([1, 2, 3, 4]))
    while Hk * r > 24:
        r -= 1
    B = int(rng.integers(1, 17))

    def batch(s):
        parents = []
        for n in rng.choice(SIZES, size=B):
            n = int(n)
            if n == 0:
                parents.append(np.zeros(0, np.int32))
            elif rng.random() < 0.2:
                parents.append(W.chain(n))
            else:
                parents.append(W.random_tree(rng, n))
        accepts = [int(rng.integers(-1, len(p))) if len(p) else -1 for p in parents]
        return W.make_custom(parents, accepts, Hv=Hk * r, Hk=Hk, seed=s)

    return batch(2 * seed), batch(2 * seed + 1)


@pytest.mark.parametrize("seed", range(10))
def test_random_shapes_one_launch_equals_two_and_the_oracle(seed):
    P, C = random_case(seed)
    res = run_pair(P, C)
    assert_same_bits(res)
    oracle_check(P, C, res)


# ---- tree attention ----------------------------------------------------------

def random_attn_case(seed):
    rng = np.random.default_rng(2000 + seed)
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    B = int(rng.integers(1, 9))
    parents = []
    for n in rng.choice(SIZES, size=B):
        n = int(n)
        parents.append(np.zeros(0, np.int32) if n == 0 else
                       (W.chain(n) if rng.random() < 0.2 else W.random_tree(rng, n)))
    ctx = [int(x) for x in rng.integers(0, 300, size=B)]
    split = [None, 64, 100, 257][int(rng.integers(0, 4))]
    return W.make_attn(parents, ctx, Hq=Hkv * G, Hkv=Hkv, seed=seed, name=f"attn_random_{seed}"), split


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_tree_attention(seed):
    """Random query/kv head ratios (1 to 16 query heads per kv head), contexts of 0-299 keys,
    trees from empty to 64 nodes, one pass or a random context split: against the oracle."""
    from test_gpu_attention import compare, oracle_attn, run_attn
    wl, split = random_attn_case(seed)
    out, lse, st, _ = run_attn(wl, split=split)
    ro, rl, rst = oracle_attn(wl)
    assert np.array_equal(st, rst)
    compare(wl, out, lse, ro, rl, [b for b in range(wl.B) if rst[b] == 0])
