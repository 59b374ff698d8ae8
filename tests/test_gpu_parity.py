"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar: bit-exact ancestry masks, accepted paths and statuses; row-normwise
relative error <= 2e-3 on node outputs, pseudo-values and committed states.
Every configuration is compared in full: the small ones in the test process,
the batch-256 ones (run whole, in the launch configuration the benchmark
times) request by request over a pool of oracle processes.  Besides the bar,
float errors must stay inside a regression envelope (helpers.ENVELOPE).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import ENVELOPE, TOL, anc_u64, host, matwise_rel_err, oracle_inputs, rowwise_rel_err, upload
import oracle_pool as OP

import speculative_decoding_tree_amd.gdn_tree as G

pytestmark = pytest.mark.gpu


def _mn(wl):
    return max(1, wl.max_nodes)


def run_gpu(wl, S0=None, state_slot=None, max_nodes=None, inplace=False):
    mn = max_nodes or _mn(wl)
    d = upload(wl, S0)
    ss = None if state_slot is None else torch.from_numpy(np.asarray(state_slot, np.int32)).cuda()
    out, U, anc, st = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"],
                               d["parent"], max_nodes=mn, state_slot=ss)
    path, plen, pst = G.accepted_path(d["node_offset"], d["parent"], d["accept_node"], max_nodes=mn)
    S_in = d["S0"].clone() if inplace else d["S0"]
    S1, cst = G.commit(S_in, U, d["k"], d["g"], d["node_offset"], d["parent"], path, plen, max_nodes=mn,
                       S_out=S_in if inplace else None, state_slot=ss)
    torch.cuda.synchronize()
    return dict(out=host(out), U=host(U), anc=anc_u64(anc), status=host(st), path=host(path),
                plen=host(plen), pstatus=host(pst), S1=host(S1), cstatus=host(cst), dev=d)


def check_full(wl, res, state_slot=None, mn=None):
    mn = mn or _mn(wl)
    Oo, Uo, anco, sto = O.verify_batch(*oracle_inputs(wl), wl.Hv, wl.Hk, max_nodes=mn, state_slot=state_slot)
    assert np.array_equal(res["status"], sto)
    assert np.array_equal(res["anc"], anco)
    ok = np.concatenate([np.arange(wl.node_offset[b], wl.node_offset[b + 1])
                         for b in range(wl.B) if sto[b] == 0] + [np.zeros(0, int)]).astype(int)
    eo = rowwise_rel_err(res["out"][ok], Oo[ok])
    eu = rowwise_rel_err(res["U"][ok], Uo[ok])
    assert eo <= TOL and eu <= TOL, (eo, eu)
    assert eo <= ENVELOPE and eu <= ENVELOPE, (eo, eu)
    po, plo, pso = O.accepted_path_batch(wl.node_offset, wl.parent, wl.accept_node, max_nodes=mn)
    assert np.array_equal(res["path"], po) and np.array_equal(res["plen"], plo)
    assert np.array_equal(res["pstatus"], pso)
    So, cso = O.commit_batch(*oracle_inputs(wl), po, plo, wl.Hv, wl.Hk, max_nodes=mn, state_slot=state_slot)
    assert np.array_equal(res["cstatus"], cso)
    es = matwise_rel_err(res["S1"], So)
    assert es <= TOL and es <= ENVELOPE, es
    for b in range(wl.B):   # nothing accepted: S0 kept bit-exactly
        slot = b if state_slot is None else state_slot[b]
        if plo[b] == 0 and cso[b] == 0:
            assert np.array_equal(res["S1"][slot], wl.S0[slot])
    return eo, eu, es


SMALL = {
    "tiny_d16_chain_pad": lambda: W.zero_pad(W.make_tiny_d16("chain")),
    "tiny_d16_tree_pad": lambda: W.zero_pad(W.make_tiny_d16("tree")),
    "chain3_b64": W.make_chain3_b64,
    "rootbranch6_b1": lambda: W.make_root_branch6(B=1),
    "rootbranch6_b16": lambda: W.make_root_branch6(B=16),
    "rootbranch6_b16_bfs": lambda: W.make_root_branch6(B=16, bfs=True),
    "mixed_small": lambda: W.make_mixed_b256(per_kind=3, Hv=6, Hk=2),
    "deep_chain64": lambda: W.make_custom([W.chain(64), W.chain(64)], [63, 20], Hv=4, Hk=2),
    "forest_empty_single": lambda: W.make_custom(
        [np.zeros(0, np.int32), np.array([-1], np.int32), np.full(8, -1, np.int32),
         np.zeros(0, np.int32), W.random_tree(np.random.default_rng(3), 40)],
        [-1, 0, 5, -1, 7], Hv=4, Hk=4),
    # 32-node build: units of one and two 16-node tiles (the K and Q grams on
    # different waves; the second tile's R rows written after a barrier)
    "nm32_mix": lambda: W.make_custom(
        [W.random_tree(np.random.default_rng(10 + s), n) for s, n in enumerate([32, 17, 1, 16, 31, 24])],
        [5, 0, 0, -1, 30, 11], Hv=6, Hk=2),
    # 16-node build with a full tile
    "nm16_full": lambda: W.make_custom(
        [W.random_tree(np.random.default_rng(20 + s), n) for s, n in enumerate([16, 1, 15, 9])],
        [15, -1, 3, 8], Hv=4, Hk=2),
    "ragged_tail_max": lambda: W.make_custom(
        [W.random_tree(np.random.default_rng(s), n) for s, n in enumerate([64, 17, 33, 5, 63, 1])],
        [3, 0, -1, 4, 10, 0], Hv=6, Hk=3),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_configs_full_parity(name):
    wl = SMALL[name]()
    res = run_gpu(wl)
    check_full(wl, res)


def test_zero_padding_is_exact():
    wl = W.zero_pad(W.make_tiny_d16("tree"))
    res = run_gpu(wl)
    assert np.all(res["out"][..., 16:] == 0) and np.all(res["U"][..., 16:] == 0)
    assert np.all(res["S1"][..., 16:, :] == 0) and np.all(res["S1"][..., :, 16:] == 0)


def test_state_slot_permutation_and_inplace_commit():
    wl = W.make_mixed_b256(per_kind=2, Hv=4, Hk=2, seed=5)
    slots = list(range(wl.B))[::-1]
    res = run_gpu(wl, state_slot=slots, inplace=True)
    check_full(wl, res, state_slot=slots)


def test_deterministic_bitwise():
    wl = W.make_mixed_b256(per_kind=2, Hv=6, Hk=2, seed=7)
    a, b = run_gpu(wl), run_gpu(wl)
    for key in ("out", "U", "S1", "anc", "path"):
        assert np.array_equal(a[key], b[key]), key


def test_sibling_perturbation_leaves_other_branches_bit_identical():
    rng = np.random.default_rng(11)
    par = W.random_tree(rng, 24)
    wl = W.make_custom([par], [5], Hv=4, Hk=2, seed=2)
    base = run_gpu(wl)
    j = 4
    sub = {t for t in range(24) if (O.ancestry(par)[t] >> j) & 1}
    wl2 = W.make_custom([par], [5], Hv=4, Hk=2, seed=2)
    wl2.v[j] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(wl2.v[j]) * 2 + 1)
    wl2.k[j] = W.f32_to_bf16_bits(-W.bf16_bits_to_f32(wl2.k[j]))
    wl2.q[j] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(wl2.q[j]) + 1)
    wl2.g[j] -= 0.5
    wl2.beta[j] = 0.9
    pert = run_gpu(wl2)
    for t in range(24):
        same = np.array_equal(base["out"][t], pert["out"][t]) and np.array_equal(base["U"][t], pert["U"][t])
        assert same == (t not in sub), t


def test_gqa_twin_heads_bit_identical():
    wl = W.make_custom([W.random_tree(np.random.default_rng(4), 20), W.chain(5)], [3, 4], Hv=4, Hk=2)
    wl.S0[:, 1] = wl.S0[:, 0]
    wl.v[:, 1] = wl.v[:, 0]
    wl.g[:, 1] = wl.g[:, 0]
    wl.beta[:, 1] = wl.beta[:, 0]
    res = run_gpu(wl)
    assert np.array_equal(res["out"][:, 0], res["out"][:, 1])
    assert np.array_equal(res["U"][:, 0], res["U"][:, 1])
    assert np.array_equal(res["S1"][:, 0], res["S1"][:, 1])


# ----------------------------------------------------------------------------
# device-detected errors
# ----------------------------------------------------------------------------

def test_device_errors():
    wl = W.make_custom([W.chain(3), W.root_branch(), W.chain(4), W.chain(2)], [2, 4, 1, -1], Hv=4, Hk=2)
    clean = run_gpu(wl)
    bad = W.make_custom([W.chain(3), W.root_branch(), W.chain(4), W.chain(2)], [2, 4, 1, -1], Hv=4, Hk=2)
    bad.parent[3 + 2] = 2                      # request 1: node 2 -> parent 2 (not < 2)
    bad.accept_node[2] = 4                     # request 2: accept beyond N
    res = run_gpu(bad)
    assert list(res["status"]) == [0, O.STATUS_BAD_PARENT, 0, 0]
    assert np.isnan(res["out"][3:9]).all() and np.isnan(res["U"][3:9]).all()
    assert np.all(res["anc"][3:9] == 0)
    for r in (slice(0, 3), slice(9, 15)):       # other requests untouched, bit-exact
        assert np.array_equal(res["out"][r], clean["out"][r])
    assert list(res["pstatus"]) == [0, O.STATUS_BAD_PARENT, O.STATUS_BAD_ACCEPT, 0]
    assert res["plen"][1] == 0 and res["plen"][2] == 0
    # commit: invalid request keeps S0; path problems give status 4 and S0
    assert np.array_equal(res["S1"][1], bad.S0[1]) and np.array_equal(res["S1"][2], bad.S0[2])
    check_full(bad, res)


def test_device_errors_paths_offsets_slots_and_node_cap():
    wl = W.make_custom([W.chain(3), W.root_branch(), W.chain(5)], [2, 4, 1], Hv=2, Hk=1)
    d = upload(wl)
    mn = 6
    # too many nodes: max_nodes 4 with requests of 6 and 5 nodes
    out, U, anc, st = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"],
                               d["parent"], max_nodes=4)
    torch.cuda.synchronize()
    assert list(host(st)) == [0, O.STATUS_TOO_MANY_NODES, O.STATUS_TOO_MANY_NODES]
    assert np.isnan(host(out)[3:]).all()
    # bad slot
    ss = torch.tensor([0, 9, 2], dtype=torch.int32, device="cuda")
    out, U, anc, st = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"],
                               d["parent"], max_nodes=mn, state_slot=ss)
    torch.cuda.synchronize()
    assert list(host(st)) == [0, O.STATUS_BAD_SLOT, 0]
    # bad offsets (request 1 ends before it starts)
    off = torch.tensor([0, 3, 2, 14], dtype=torch.int32, device="cuda")
    out, U, anc, st = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], off, d["parent"],
                               max_nodes=mn)
    torch.cuda.synchronize()
    assert host(st)[1] == O.STATUS_BAD_OFFSETS
    # bad paths: not a chain / too long / negative length
    out, U, anc, st = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"],
                               d["parent"], max_nodes=mn)
    path = torch.zeros((3, mn), dtype=torch.int32, device="cuda")
    path[0, :2] = torch.tensor([0, 2])
    path[1, :3] = torch.tensor([3, 4, 5])
    plen = torch.tensor([2, 3, 7], dtype=torch.int32, device="cuda")
    S_out = torch.zeros_like(d["S0"])
    S1, cst = G.commit(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"], path, plen, max_nodes=mn,
                       S_out=S_out)
    torch.cuda.synchronize()
    assert list(host(cst)) == [O.STATUS_BAD_PATH, 0, O.STATUS_BAD_PATH]
    S1 = host(S1)
    assert np.array_equal(S1[0], wl.S0[0]) and np.array_equal(S1[2], wl.S0[2])
    So, cso = O.commit_batch(*oracle_inputs(wl), host(path), host(plen), wl.Hv, wl.Hk, max_nodes=mn,
                             S_out_init=np.zeros_like(wl.S0))
    assert list(cso) == list(host(cst))
    assert matwise_rel_err(S1, So) <= TOL


# ----------------------------------------------------------------------------
# storeall comparison variant
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["chain3_b64", "rootbranch6_b16", "mixed_small", "forest_empty_single"])
def test_storeall_parity(name):
    wl = SMALL[name]()
    if name == "chain3_b64":
        wl = W.subset(wl, range(16))
    mn = _mn(wl)
    d = upload(wl)
    out, NS, st = G.verify_storeall(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"],
                                    d["parent"], max_nodes=mn)
    S1, cst = G.commit_storeall(d["S0"], NS, d["node_offset"], d["parent"], d["accept_node"], max_nodes=mn)
    torch.cuda.synchronize()
    Oo, NSo, sto = O.verify_storeall_batch(*oracle_inputs(wl), wl.Hv, wl.Hk, max_nodes=mn)
    assert np.array_equal(host(st), sto)
    assert rowwise_rel_err(host(out), Oo) <= TOL
    assert matwise_rel_err(host(NS), NSo) <= TOL
    So, cso = O.commit_storeall_batch(wl.S0, NSo, wl.node_offset, wl.parent, wl.accept_node, max_nodes=mn)
    assert np.array_equal(host(cst), cso)
    assert matwise_rel_err(host(S1), So) <= TOL


# ----------------------------------------------------------------------------
# batch-256 configurations, whole batch on the GPU, sampled oracle
# ----------------------------------------------------------------------------

def full_batch_check(wl, res):
    """Statuses, masks and paths in full; out, U and S' of every request against the
    oracle, evaluated one request per task over a process pool."""
    mn = _mn(wl)
    assert np.all(res["status"] == 0) and np.all(res["cstatus"] == 0) and np.all(res["pstatus"] == 0)
    anc = np.concatenate([np.array(O.ancestry(wl.parents_of(b)), dtype=np.uint64) for b in range(wl.B)])
    assert np.array_equal(res["anc"], anc)
    po, plo, _ = O.accepted_path_batch(wl.node_offset, wl.parent, wl.accept_node, max_nodes=mn)
    assert np.array_equal(res["path"], po) and np.array_equal(res["plen"], plo)
    arrays = OP.workload_arrays(wl)
    arrays.update(out=res["out"], U=res["U"], S1=res["S1"])
    rows = OP.run(arrays, OP.verify_commit_request, [(b, wl.Hv, wl.Hk) for b in range(wl.B)])
    assert sorted(r[0] for r in rows) == list(range(wl.B)) and all(r[1] == 0 for r in rows)
    worst = [max(r[k] for r in rows) for k in (2, 3, 4)]
    print(f"{wl.name}: all {wl.B} requests, worst rel err out/U/S': {worst}")
    assert max(worst) <= TOL, worst
    assert max(worst) <= ENVELOPE, worst
    return worst


def test_random32_b256_full_batch_every_request():
    wl = W.make_random32_b256()
    res = run_gpu(wl)
    full_batch_check(wl, res)


def test_mixed_b256_full_batch_every_request():
    wl = W.make_mixed_b256()
    res = run_gpu(wl)
    full_batch_check(wl, res)


def test_commit_alone_from_oracle_pseudo_values():
    """commit fed with the oracle's U (cast to fp32): isolates the commit kernel."""
    wl = SMALL["mixed_small"]()
    mn = _mn(wl)
    Oo, Uo, _, _ = O.verify_batch(*oracle_inputs(wl), wl.Hv, wl.Hk, max_nodes=mn)
    d = upload(wl)
    U = torch.from_numpy(Uo.astype(np.float32)).cuda()
    po, plo, _ = O.accepted_path_batch(wl.node_offset, wl.parent, wl.accept_node, max_nodes=mn)
    S1, cst = G.commit(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"],
                       torch.from_numpy(po).cuda(), torch.from_numpy(plo).cuda(), max_nodes=mn)
    torch.cuda.synchronize()
    So, _ = O.commit_batch(*oracle_inputs(wl), po, plo, wl.Hv, wl.Hk, max_nodes=mn)
    assert matwise_rel_err(host(S1), So) <= 1e-5


# ----------------------------------------------------------------------------
# device-side greedy acceptance, alone and fused with the commit
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["chain3_b64", "rootbranch6_b16", "mixed_small", "forest_empty_single", "deep_chain64"])
def test_greedy_accept_and_fused_commit(name):
    wl = SMALL[name]()
    mn = _mn(wl)
    draft, tgt, root = W.greedy_tokens(wl, p_match=0.8, seed=3)
    acc_o, path_o, plen_o, st_o = O.greedy_accept_batch(wl.node_offset, wl.parent, draft, tgt, root, max_nodes=mn)
    d = upload(wl)
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    acc, path, plen, st = G.accept_greedy(d["node_offset"], d["parent"], tt(draft), tt(tgt), tt(root), max_nodes=mn)
    out, U, _, _ = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"],
                            max_nodes=mn)
    S1, acc2, path2, plen2, st2 = G.accept_commit(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"],
                                                  tt(draft), tt(tgt), tt(root), max_nodes=mn)
    torch.cuda.synchronize()
    for got in ((acc, path, plen, st), (acc2, path2, plen2, st2)):
        assert np.array_equal(host(got[0]), acc_o)
        assert np.array_equal(host(got[1]), path_o) and np.array_equal(host(got[2]), plen_o)
        assert np.array_equal(host(got[3]), st_o)
    So, _ = O.commit_batch(*oracle_inputs(wl), path_o, plen_o, wl.Hv, wl.Hk, max_nodes=mn)
    assert matwise_rel_err(host(S1), So) <= TOL
    # the fused launch equals verify -> accepted path -> commit bit for bit
    S3, _ = G.commit(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"], path, plen, max_nodes=mn)
    torch.cuda.synchronize()
    assert np.array_equal(host(S3), host(S1))


def test_fused_accept_commit_full_batch():
    wl = W.make_mixed_b256()
    mn = wl.max_nodes
    draft, tgt, root = W.greedy_tokens(wl)
    acc_o, path_o, plen_o, _ = O.greedy_accept_batch(wl.node_offset, wl.parent, draft, tgt, root, max_nodes=mn)
    d = upload(wl)
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    out, U, _, _ = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"],
                            max_nodes=mn)
    S1, acc, path, plen, st = G.accept_commit(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"],
                                              tt(draft), tt(tgt), tt(root), max_nodes=mn)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), acc_o) and np.array_equal(host(path), path_o)
    assert np.array_equal(host(plen), plen_o) and np.all(host(st) == 0)
    rng = np.random.default_rng(1)
    S1h = host(S1)
    for b in sorted(rng.choice(wl.B, 12, replace=False).tolist()):
        lo, hi = wl.node_offset[b], wl.node_offset[b + 1]
        pth = O.accepted_path(wl.parents_of(b), int(acc_o[b]))
        for h in range(0, wl.Hv, 7):
            want = O.replay_commit_unit(wl.S0[b, h], wl.q64()[lo:hi, h // 3], wl.k64()[lo:hi, h // 3],
                                        wl.v64()[lo:hi, h], wl.g[lo:hi, h].astype(np.float64),
                                        wl.beta[lo:hi, h].astype(np.float64), pth)
            assert matwise_rel_err(S1h[b, h][None], want[None]) <= TOL


@pytest.mark.parametrize("name", ["rootbranch6_b16", "mixed_small", "deep_chain64", "forest_empty_single"])
def test_commit_node_equals_accepted_path_then_commit(name):
    """The fused launch derives the same path and writes the same state, bit for bit."""
    wl = SMALL[name]()
    mn = _mn(wl)
    d = upload(wl)
    _, U, _, _ = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"],
                          max_nodes=mn)
    path, plen, pst = G.accepted_path(d["node_offset"], d["parent"], d["accept_node"], max_nodes=mn)
    S_ref, cst = G.commit(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"], path, plen, max_nodes=mn)
    S1, path1, plen1, st1 = G.commit_node(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"],
                                          d["accept_node"], max_nodes=mn)
    torch.cuda.synchronize()
    assert np.array_equal(host(S1), host(S_ref))
    assert np.array_equal(host(path1), host(path)) and np.array_equal(host(plen1), host(plen))
    assert np.array_equal(host(st1), host(cst))
    po, plo, _ = O.accepted_path_batch(wl.node_offset, wl.parent, wl.accept_node, max_nodes=mn)
    assert np.array_equal(host(path1), po) and np.array_equal(host(plen1), plo)


def test_commit_node_bad_accept_node_keeps_S0():
    wl = W.make_root_branch6(4)
    mn = wl.max_nodes
    d = upload(wl)
    _, U, _, _ = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"],
                          max_nodes=mn)
    acc = torch.tensor([2, 6, -2, -1], dtype=torch.int32, device=d["S0"].device)   # 6 and -2 are out of range
    S1, path, plen, st = G.commit_node(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"], acc,
                                       max_nodes=mn)
    torch.cuda.synchronize()
    st, S1h, S0h = host(st), host(S1), wl.S0
    assert list(st) == [O.STATUS_OK, O.STATUS_BAD_ACCEPT, O.STATUS_BAD_ACCEPT, O.STATUS_OK]
    for b in (1, 2, 3):                                   # bad node, bad node, nothing accepted: S' = S0
        assert np.array_equal(S1h[b], S0h[b])
    assert list(host(plen)) == [3, 0, 0, 0]
    assert (host(path)[1:] == 0).all()


# ----------------------------------------------------------------------------
# replay commit (no pseudo-values)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["chain3_b64", "rootbranch6_b16", "mixed_small", "deep_chain64", "forest_empty_single"])
def test_commit_replay_parity(name):
    wl = SMALL[name]()
    mn = _mn(wl)
    d = upload(wl)
    po, plo, _ = O.accepted_path_batch(wl.node_offset, wl.parent, wl.accept_node, max_nodes=mn)
    path, plen = torch.from_numpy(po).cuda(), torch.from_numpy(plo).cuda()
    S1, st = G.commit_replay(d["S0"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"], path,
                             plen, max_nodes=mn)
    out, U, _, _ = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"],
                            max_nodes=mn)
    S2, _ = G.commit(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"], path, plen, max_nodes=mn)
    torch.cuda.synchronize()
    So, cso = O.commit_batch(*oracle_inputs(wl), po, plo, wl.Hv, wl.Hk, max_nodes=mn)
    assert np.array_equal(host(st), cso)
    assert matwise_rel_err(host(S1), So) <= TOL
    assert matwise_rel_err(host(S1), host(S2).astype(np.float64)) <= TOL
    for b in range(wl.B):
        if plo[b] == 0:
            assert np.array_equal(host(S1)[b], wl.S0[b])


def test_commit_replay_inplace_and_bad_path():
    wl = W.make_custom([W.chain(3), W.root_branch()], [2, 4], Hv=2, Hk=1)
    d = upload(wl)
    path = torch.tensor([[0, 1, 2, 0, 0, 0], [0, 2, 0, 0, 0, 0]], dtype=torch.int32, device="cuda")
    plen = torch.tensor([3, 2], dtype=torch.int32, device="cuda")
    S = d["S0"].clone()
    S1, st = G.commit_replay(S, d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"], path, plen,
                             max_nodes=6, S_out=S)
    torch.cuda.synchronize()
    assert list(host(st)) == [0, O.STATUS_BAD_PATH]
    So, _ = O.commit_batch(*oracle_inputs(wl), host(path), host(plen), wl.Hv, wl.Hk, max_nodes=6)
    assert matwise_rel_err(host(S1)[:1], So[:1]) <= TOL
    assert np.array_equal(host(S1)[1], wl.S0[1])


# ----------------------------------------------------------------------------
# load-adaptive budget selection
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("budget_frac,thr", [(0.0, 0.0), (0.1, 0.0), (0.5, 0.05), (0.9, 0.3), (1.2, 0.0)])
def test_budget_select_bit_exact(budget_frac, thr):
    wl = W.make_mixed_b256(per_kind=8, Hv=2, Hk=1, seed=4)
    p = W.acceptance_probs(wl, seed=5)
    p[::11] = 1.0                                    # exact survival ties along paths
    budget = int(budget_frac * wl.T)
    so, ko, co, sto = O.budget_select(wl.node_offset, wl.parent, p, budget, thr)
    d = upload(wl)
    s, keep, kept, st = G.budget_select(d["node_offset"], d["parent"], torch.from_numpy(p).cuda(), budget, thr,
                                        max_nodes=wl.max_nodes)
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(keep), ko) and np.array_equal(host(kept), co) and np.array_equal(host(st), sto)


def test_budget_select_invalid_request_and_full_batch():
    wl = W.make_mixed_b256()
    p = W.acceptance_probs(wl)
    par = wl.parent.copy()
    par[wl.node_offset[7] + 1] = 5                   # request 7 breaks parent order
    so, ko, co, sto = O.budget_select(wl.node_offset, par, p, wl.T // 3, 0.01)
    assert sto[7] == O.STATUS_BAD_PARENT
    d = upload(wl)
    s, keep, kept, st = G.budget_select(d["node_offset"], torch.from_numpy(par).cuda(), torch.from_numpy(p).cuda(),
                                        wl.T // 3, 0.01, max_nodes=wl.max_nodes)
    torch.cuda.synchronize()
    sh = host(s)
    assert np.array_equal(np.isnan(sh), np.isnan(so))
    ok = ~np.isnan(so)
    assert np.array_equal(sh[ok].view(np.uint32), so[ok].view(np.uint32))
    assert np.array_equal(host(keep), ko) and np.array_equal(host(kept), co) and np.array_equal(host(st), sto)


@pytest.mark.parametrize("budget_frac", [0.1, 0.6])
def test_budget_select_more_nodes_than_register_cache(budget_frac):
    # 160 random 64-node trees: 10240 nodes, more than the 8192 keys the select
    # kernel keeps in registers, so every radix pass re-reads them
    rng = np.random.default_rng(31)
    parents = [W.random_tree(rng, 64) for _ in range(160)]
    wl = W.make_custom(parents, [0] * len(parents), Hv=1, Hk=1, seed=32)
    assert wl.T > 8192
    p = W.acceptance_probs(wl, seed=33)
    budget = int(budget_frac * wl.T)
    so, ko, co, sto = O.budget_select(wl.node_offset, wl.parent, p, budget, 0.02)
    d = upload(wl)
    s, keep, kept, st = G.budget_select(d["node_offset"], d["parent"], torch.from_numpy(p).cuda(), budget, 0.02,
                                        max_nodes=wl.max_nodes)
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(keep), ko) and np.array_equal(host(kept), co) and np.array_equal(host(st), sto)


def test_budget_select_tie_order_hand_cases():
    """The hand-built tie cases (tests/golden/budget_ties.json): the kernel's keep sets
    equal the ones written out by hand, bit for bit."""
    import json
    import os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "budget_ties.json")))["cases"]
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    for c in cases:
        B = len(c["node_offset"]) - 1
        s, keep, kept, st = G.budget_select(i32(c["node_offset"]), i32(c["parent"]),
                                            torch.tensor(c["p"], dtype=torch.float32, device="cuda"),
                                            c["budget"], c["threshold"], max_nodes=8)
        torch.cuda.synchronize()
        assert host(st).tolist() == [0] * B, c["name"]
        assert host(keep).tolist() == c["expected_keep"], c["name"]
        assert host(kept).tolist() == c["expected_kept"], c["name"]


# ----------------------------------------------------------------------------
# non-finite inputs stay inside their subtree
# ----------------------------------------------------------------------------

def _nonfinite_workload():
    rng = np.random.default_rng(41)
    # a 16-node build tree, a 32-node build tree and a 64-node build tree in one batch
    return W.make_custom([W.root_branch(), W.random_tree(rng, 24), W.random_tree(rng, 64)], [2, 5, 9],
                         Hv=4, Hk=2, seed=42)


def _perturb(wl, kind, b, j):
    """NaN gate, NaN beta or Inf value entries of node j of request b (every head)."""
    t = int(wl.node_offset[b]) + j
    if kind == "nan_g":
        wl.g[t] = np.nan
    elif kind == "nan_beta":
        wl.beta[t] = np.nan
    else:
        wl.v[t, :, 5] = 0x7F80        # +Inf in bf16, value column 5
        wl.v[t, 1, 77] = 0xFF80       # -Inf, head 1, column 77
    return t


def _check_nonfinite(wl_clean, wl_bad, clean, bad, sub_rows):
    """Rows outside the perturbed subtree keep their bits; inside it the device is
    non-finite exactly where the oracle is, and finite entries meet the bar."""
    T = wl_clean.T
    outside = np.setdiff1d(np.arange(T), sub_rows)
    for key in ("out", "U"):
        assert np.array_equal(clean[key][outside].view(np.uint32), bad[key][outside].view(np.uint32)), key
    with np.errstate(invalid="ignore", over="ignore"):
        Oo, Uo, anco, sto = O.verify_batch(*oracle_inputs(wl_bad), wl_bad.Hv, wl_bad.Hk, max_nodes=_mn(wl_bad))
    for key, ref in (("out", Oo), ("U", Uo)):
        got, want = bad[key][sub_rows].astype(np.float64), ref[sub_rows]
        assert np.array_equal(np.isfinite(got), np.isfinite(want)), key
        fin = np.isfinite(want)
        scale = np.abs(np.where(fin, want, 0)).max(axis=-1, keepdims=True)
        with np.errstate(invalid="ignore"):   # got - want is NaN where both are (those entries are masked)
            err = np.abs(np.where(fin, got - want, 0)) / np.maximum(scale, 1e-30)
        assert err.max() <= TOL, (key, err.max())


@pytest.mark.parametrize("kind", ["nan_g", "nan_beta", "inf_v"])
def test_non_finite_sibling_stays_in_subtree(kind):
    """TreeWY, Method: a branch reads only its ancestors.  A NaN or Inf in one node's g, beta
    or v reaches its subtree only; the other branches keep their bits (verify), and the
    commit of a path that avoids the node keeps its bits as well."""
    wl = _nonfinite_workload()
    clean = run_gpu(wl)
    wl2 = _nonfinite_workload()
    for b, j in ((0, 3), (1, 4), (2, 1)):
        _perturb(wl2, kind, b, j)
    bad = run_gpu(wl2)
    sub_rows = []
    for b, j in ((0, 3), (1, 4), (2, 1)):
        lo = int(wl.node_offset[b])
        anc = O.ancestry(wl.parents_of(b))
        sub_rows += [lo + t for t in range(wl.nodes(b)) if (anc[t] >> j) & 1]
    sub_rows = np.array(sorted(sub_rows))
    _check_nonfinite(wl, wl2, clean, bad, sub_rows)
    assert np.array_equal(clean["anc"], bad["anc"]) and np.array_equal(clean["status"], bad["status"])
    # commits whose accepted path avoids every perturbed node keep their bits
    for b, j in ((0, 3), (1, 4), (2, 1)):
        path = O.accepted_path(wl.parents_of(b), int(wl.accept_node[b]))
        if j not in path:
            assert np.array_equal(clean["S1"][b].view(np.uint32), bad["S1"][b].view(np.uint32)), b


@pytest.mark.parametrize("kind", ["nan_g", "inf_v"])
def test_non_finite_stays_in_subtree_storeall_and_replay(kind):
    """The snapshot-per-node verify and the replay commit walk the sequential rule, so a
    non-finite input of one node reaches only its subtree there too: every other node's output
    and state, and the replay commit of a path that avoids the node, keep their bits."""
    perturbed = ((0, 3), (1, 4), (2, 1))
    wl, wl2 = _nonfinite_workload(), _nonfinite_workload()
    for b, j in perturbed:
        _perturb(wl2, kind, b, j)
    mn = _mn(wl)
    res = {}
    for tag, w in (("clean", wl), ("bad", wl2)):
        d = upload(w)
        out, NS, st = G.verify_storeall(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"],
                                        d["parent"], max_nodes=mn)
        path, plen, _ = G.accepted_path(d["node_offset"], d["parent"], d["accept_node"], max_nodes=mn)
        S2, rst = G.commit_replay(d["S0"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"],
                                  path, plen, max_nodes=mn)
        torch.cuda.synchronize()
        res[tag] = dict(out=host(out), NS=host(NS), st=host(st), S2=host(S2), rst=host(rst))
    assert (res["clean"]["st"] == 0).all() and (res["bad"]["st"] == 0).all() and (res["bad"]["rst"] == 0).all()
    sub_rows = []
    for b, j in perturbed:
        lo = int(wl.node_offset[b])
        anc = O.ancestry(wl.parents_of(b))
        sub_rows += [lo + t for t in range(wl.nodes(b)) if (anc[t] >> j) & 1]
    outside = np.setdiff1d(np.arange(wl.T), sub_rows)
    for key in ("out", "NS"):
        assert np.array_equal(res["clean"][key][outside].view(np.uint32), res["bad"][key][outside].view(np.uint32)), key
        assert not np.isfinite(res["bad"][key][sub_rows]).all(), key
    for b, j in perturbed:
        path = O.accepted_path(wl.parents_of(b), int(wl.accept_node[b]))
        if j not in path:
            assert np.array_equal(res["clean"]["S2"][b].view(np.uint32), res["bad"]["S2"][b].view(np.uint32)), b
        else:
            assert not np.isfinite(res["bad"]["S2"][b]).all(), b


def test_non_finite_pseudo_value_off_the_path_does_not_reach_the_commit():
    """The commit reads only the accepted path's pseudo-values: NaN and Inf rows of
    other nodes leave S' bit-identical (gdn_tree_commit_node and gdn_tree_commit)."""
    wl = _nonfinite_workload()
    mn = _mn(wl)
    d = upload(wl)
    _, U, _, _ = G.verify(d["S0"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["node_offset"], d["parent"],
                          max_nodes=mn)
    S_ref, path, plen, _ = G.commit_node(d["S0"], U, d["k"], d["g"], d["node_offset"], d["parent"],
                                         d["accept_node"], max_nodes=mn)
    torch.cuda.synchronize()
    U2 = U.clone()
    for b in range(wl.B):
        on_path = set(host(path)[b, :int(host(plen)[b])].tolist())
        lo = int(wl.node_offset[b])
        off = [t for t in range(wl.nodes(b)) if t not in on_path]
        U2[lo + off[0]] = float("nan")
        U2[lo + off[-1], :, 3] = float("inf")
    S1, _, _, st = G.commit_node(d["S0"], U2, d["k"], d["g"], d["node_offset"], d["parent"], d["accept_node"],
                                 max_nodes=mn)
    S2, st2 = G.commit(d["S0"], U2, d["k"], d["g"], d["node_offset"], d["parent"], path, plen, max_nodes=mn)
    torch.cuda.synchronize()
    assert torch.equal(S1.view(torch.int32), S_ref.view(torch.int32))
    assert torch.equal(S2.view(torch.int32), S_ref.view(torch.int32))
    assert (host(st) == 0).all() and (host(st2) == 0).all()


def test_16node_build_at_batch256_grid_every_request():
    """The 16-node build on a batch-256 grid (its index arithmetic is emulated on the CPU in
    test_verify_index_bounds.py): 128 depth-3 chains and 128 root-branch trees, 32 value /
    16 key heads, every request against the oracle."""
    rng = np.random.default_rng(51)
    parents = [W.chain(3) if b % 2 else W.root_branch() for b in range(256)]
    accepts = [int(rng.integers(-1, len(p))) for p in parents]
    wl = W.make_custom(parents, accepts, Hv=32, Hk=16, seed=52, name="chain3_rootbranch6_b256")
    assert wl.max_nodes <= 16
    res = run_gpu(wl)
    full_batch_check(wl, res)
