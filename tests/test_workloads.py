"""Seeded synthetic input generators: determinism, shapes and distributions."""
import numpy as np
import pytest

import workloads as W


def test_bf16_round_trip_and_ties():
    x = np.array([1.0, -2.5, 3.14159, 1e-3, 65504.0], np.float32)
    b = W.f32_to_bf16_bits(x)
    y = W.bf16_bits_to_f32(b)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)
    # exactly-representable values survive, ties round to even
    assert W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.array([1.5], np.float32)))[0] == 1.5
    tie = np.array([0x3F808000], np.uint32).view(np.float32)      # 1.00390625: halfway
    assert W.f32_to_bf16_bits(tie)[0] == 0x3F80


@pytest.mark.parametrize("name", ["tiny_d16_chain", "tiny_d16_tree", "chain3_b64", "rootbranch6_b1", "rootbranch6_b16"])
def test_deterministic(name):
    a, b = W.make(name), W.make(name)
    for f in ("node_offset", "parent", "accept_node", "S0", "q", "k", "v", "g", "beta"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_c2_shapes_and_distributions():
    wl = W.make("chain3_b64")
    assert (wl.B, wl.Hv, wl.Hk, wl.d, wl.T) == (64, 32, 16, 128, 192)
    assert wl.S0.shape == (64, 32, 128, 128) and wl.S0.dtype == np.float32
    assert abs(wl.S0.std() - np.sqrt(0.02)) < 1e-3
    kn = np.linalg.norm(W.bf16_bits_to_f32(wl.k).astype(np.float64), axis=-1)
    assert np.all(np.abs(kn - 1) < 2 ** -7)
    assert np.all(wl.g <= 0) and np.all((wl.beta > 0) & (wl.beta < 1))
    assert set(wl.accept_node.tolist()) <= {-1, 0, 1, 2}


def test_random_tree_depth_cap():
    rng = np.random.default_rng(0)
    for n in (16, 32, 64):
        for _ in range(50):
            p = W.random_tree(rng, n)
            assert all(-1 <= p[i] < i for i in range(n))
            assert W.tree_depths(p).max() <= 6


def test_c5_composition():
    wl = W.make_mixed_b256(per_kind=8, Hv=6, Hk=2)
    assert wl.B == 32
    from collections import Counter
    assert Counter(wl.kinds) == {k: 8 for k in W.MIXED_KINDS}
    sizes = {"chain3": 3, "rootbranch6": 6, "random16": 16, "random64": 64}
    for b, kd in enumerate(wl.kinds):
        assert wl.nodes(b) == sizes[kd]


def test_accept_by_edge_probabilities():
    rng = np.random.default_rng(1)
    ch = W.chain(3)
    L = [W.accept_by_edge(rng, ch) + 1 for _ in range(20000)]
    assert abs(np.mean(L) - (0.7 + 0.49 + 0.343)) < 0.03


def test_zero_pad_and_subset():
    wl = W.make_tiny_d16("tree")
    p = W.zero_pad(wl)
    assert p.d == 128 and p.S0.dtype == np.float32
    assert np.all(p.S0[:, :, 16:, :] == 0) and np.all(W.bf16_bits_to_f32(p.q)[:, :, 16:] == 0)
    c = W.make_custom([W.chain(2), W.chain(3), W.root_branch()], [0, 1, 2], Hv=2, Hk=1, d=8)
    s = W.subset(c, [2, 0])
    assert s.B == 2 and s.T == 8 and np.array_equal(s.parent[:6], W.root_branch())
    assert np.array_equal(s.S0[1], c.S0[0])
