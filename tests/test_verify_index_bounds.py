"""CPU emulation of the verify kernels' index arithmetic at batch-256 grids.

The address expressions of speculative_decoding_tree_amd/csrc/verify.hip (the
workgroup -> unit deal of common.h, every global load and store, every LDS
offset) are evaluated here for every workgroup and thread of a launch, in
numpy, and checked against the buffer and LDS sizes.  Cases: depth-3 chains
and 6-node root-branch trees at batch 256 with 32 value / 16 key heads (the
16-node build), the random 32-node batch (32-node build) and the mixed batch
(64-node build), in the verify mode and in the one-launch commit + verify
mode with the same tree as the previous one.  A second test compiles every
kernel of the library and checks that none uses scratch memory or spills
registers.
"""
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import workloads as W

D = 128
NT = 256
PCHUNK = 16


def xcd_group_unit(w, B, Hk, r):
    """common.h xcd_group_unit, vectorised over workgroup ids w."""
    cs = 1 if Hk % 16 == 0 else 0
    x, s = w & 7, w >> 3
    qi, j = s // r, s % r
    ch, wi = qi >> cs, qi - ((qi >> cs) << cs)
    q = ((ch * 8 + x) << cs) + wi
    return np.where(q < B * Hk, q * r + j, -1)


def xcd_group_grid(B, Hk, r):
    C = 2 if Hk % 16 == 0 else 1
    return 8 * ((B * Hk + 8 * C - 1) // (8 * C)) * C * r


def build_nm(max_nodes):
    return 16 if max_nodes <= 16 else (32 if max_nodes <= 32 else 64)


class Bounds:
    """Collects (name, lowest index, highest index + 1, size) of every access."""

    def __init__(self):
        self.seen = {}

    def check(self, name, lo_idx, hi_idx, size):
        lo_idx, hi_idx = int(np.min(lo_idx)), int(np.max(hi_idx))
        assert lo_idx >= 0, (name, lo_idx)
        assert hi_idx <= size, (name, hi_idx, size)
        a, b, _ = self.seen.get(name, (lo_idx, hi_idx, size))
        self.seen[name] = (min(a, lo_idx), max(b, hi_idx), size)


def emulate(wl, mode, prev=None):
    """Every global and LDS access of one launch of verify_kernel<NM, mode>."""
    B, Hv, Hk, T = wl.B, wl.Hv, wl.Hk, wl.T
    r = Hv // Hk
    NM = build_nm(wl.max_nodes)
    KT = NM // 16
    n_slots = B
    RU_BYTES = NM * (D + 2) * 4
    KOFF = RU_BYTES - NM * 2 * D
    chk = Bounds()
    grid = xcd_group_grid(B, Hk, r)
    units = xcd_group_unit(np.arange(grid), B, Hk, r)
    live = units[units >= 0]
    # the deal is a bijection onto the (request, v-head) units
    assert np.array_equal(np.sort(live), np.arange(B * Hv))
    tid = np.arange(NT)
    lane, wv = tid & 63, tid >> 6
    n, grp = lane & 15, lane >> 4
    c = 32 * wv + 2 * n
    srow, sch = tid >> 4, tid & 15
    off = wl.node_offset.astype(np.int64)
    nodes = np.diff(off)
    depth = np.concatenate([W.tree_depths(wl.parents_of(b)) for b in range(B)]) if T else np.zeros(0, int)
    for unit in live:
        b, h = int(unit) // Hv, int(unit) % Hv
        hk = h // r
        lo, N = int(off[b]), int(nodes[b])
        slot = b
        # H0 reads (and, in the fused modes, the S_out stores at the same places)
        hoff = (slot * Hv + h) * D * D + 8 * grp * D + c
        s_e = (32 * np.arange(4)[:, None] + np.arange(8)[None, :]).ravel() * D
        idx = hoff[:, None] + s_e[None, :]
        chk.check("S0 / S_out float2", idx, idx + 2, n_slots * Hv * D * D)
        if mode != 0 and prev is not None:
            plo, PN = int(prev.node_offset[b]), int(prev.node_offset[b + 1] - prev.node_offset[b])
            if PN > 0:
                tc = np.minimum(lane[wv == 1], PN - 1)
                chk.check("parent_prev", plo + tc, plo + tc + 1, prev.T)
                chk.check("g_prev", (plo + tc) * Hv + h, (plo + tc) * Hv + h + 1, prev.T * Hv)
            acc = int(prev.accept_node[b])
            path = [] if acc < 0 else _root_to(prev.parents_of(b), acc)
            L = len(path)
            chk.check("path_out row", b * prev.max_nodes + np.arange(max(L, 1)) * (L > 0),
                      b * prev.max_nodes + max(L, 1) * (L > 0) + (L == 0) * 0, B * prev.max_nodes)
            chk.check("path_out fill", b * prev.max_nodes + L, b * prev.max_nodes + prev.max_nodes,
                      B * prev.max_nodes)
            chk.check("cpath / ccoef", 0, max(L, 0), 64)
            e0 = 8 * (tid & 15)
            for j0 in range(0, L, PCHUNK):
                nj = min(PCHUNK, L - j0)
                q = j0 + np.minimum(srow, nj - 1)
                t = np.array(path)[q]
                assert (t < PN).all()
                kidx = ((plo + t) * Hk + hk) * D + e0
                chk.check("k_prev 16 bytes", kidx, kidx + 8, prev.T * Hk * D)
                uidx = ((plo + t) * Hv + h) * D + e0
                chk.check("U_prev 2 x float4", uidx, uidx + 8, prev.T * Hv * D)
                chk.check("LDS prow rows", srow, PCHUNK + srow + 1, 2 * PCHUNK)
                chk.check("LDS prow columns", e0, e0 + 8, D)
                chk.check("LDS prow reads", 32 * np.arange(4)[:, None] + 8 * grp[None, :],
                          32 * np.arange(4)[:, None] + 8 * grp[None, :] + 8, D)
                chk.check("LDS prow u reads", c, c + 2, D)
        if N == 0:
            continue
        nkt = (N + 15) >> 4
        assert nkt <= KT
        krow = Hk * D
        kbase = (lo * Hk + hk) * D
        for tau in range(nkt):
            rows = np.minimum(16 * tau + srow, N - 1)
            byte = kbase * 2 + rows * krow * 2 + 16 * sch
            chk.check("q / k staged 16 bytes", byte, byte + 16, T * Hk * D * 2)
            for i in range(4):
                vr = np.minimum(16 * tau + 4 * grp + i, N - 1)
                vidx = (lo * Hv + h) * D + vr * Hv * D + c
                chk.check("v 32-bit", vidx, vidx + 2, T * Hv * D)
            # LDS staging (Q rows from the start of the R/U area, K rows at its end)
            row = 16 * tau + srow
            so = row * 2 * D + ((sch ^ (row & 15)) << 4)
            chk.check("LDS staged Q", so, so + 16, KOFF)
            chk.check("LDS staged K", KOFF + so, KOFF + so + 16, RU_BYTES)
            # fragment reads: rows 16 tau + n, chunks 4 s + grp
            frow = 16 * tau + n
            fo = frow[:, None] * 2 * D + (((4 * np.arange(4)[None, :] + grp[:, None]) ^ (frow[:, None] & 15)) << 4)
            chk.check("LDS fragment Q", fo, fo + 16, KOFF)
            chk.check("LDS fragment K", KOFF + fo, KOFF + fo + 16, RU_BYTES)
            # R rows and the row vectors read as float4
            r0 = 16 * tau + 4 * grp
            chk.check("LDS ru rows", r0, r0 + 4, NM)
            chk.check("LDS ru columns", c, c + 2, D + 2)
            chk.check("LDS beta float4", r0, r0 + 4, 64)
            chk.check("LDS G2 / gam float4", r0, r0 + 4, NM)
        tc = np.minimum(lane, N - 1)
        chk.check("parent", lo + tc, lo + tc + 1, T)
        chk.check("g / beta", (lo + tc) * Hv + h, (lo + tc) * Hv + h + 1, T * Hv)
        chk.check("anc_mask", lo, lo + N, T)
        # grams: table entries T[r][dep(j) - 1] and T[j][r]
        dmax = int(depth[lo:lo + N].max())
        chk.check("LDS coefficient table A", 0, dmax, NM + 2)
        chk.check("LDS coefficient table P", 0, N, NM)
        chk.check("LDS level starts", 1, dmax + 2, NM + 2)
        # solve and output stores
        t = np.arange(N)
        uidx = (lo * Hv + h) * D + c[:, None] + t[None, :] * Hv * D
        chk.check("U / out float2 stores", uidx, uidx + 2, T * Hv * D)
        # output product: rows j0, j0 + 1 of ru and T, clamped to 0 past the table
        nks = (N + 31) >> 5
        for ks in range(nks):
            j0 = 32 * ks + 8 * grp[:, None] + 2 * np.arange(4)[None, :]
            jr = np.where(j0 < NM, j0, 0)
            chk.check("LDS output rows", jr, jr + 2, NM)
            for tau in range(nkt):
                chk.check("LDS output table column", 16 * tau + n, 16 * tau + n + 1, NM + 2)
        # the error path's NaN rows
        chk.check("NaN rows", (lo * Hv + h) * D, ((lo + N - 1) * Hv + h) * D + D, T * Hv * D)
    return chk.seen


def _root_to(par, t):
    path = []
    while t >= 0:
        path.append(t)
        t = int(par[t])
    return path[::-1]


CASES = {
    "chain3_b256_16node": lambda: W.make_custom([W.chain(3)] * 256, [2] * 256, Hv=32, Hk=16, seed=1),
    "rootbranch6_b256_16node": lambda: W.make_custom([W.root_branch()] * 256, [5] * 256, Hv=32, Hk=16, seed=2),
    "random32_b256_32node": W.make_random32_b256,
    "mixed_b256_64node": W.make_mixed_b256,
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("mode", [0, 1])
def test_verify_index_arithmetic_in_bounds(name, mode):
    wl = CASES[name]()
    seen = emulate(wl, mode, prev=wl if mode else None)
    assert "S0 / S_out float2" in seen and "U / out float2 stores" in seen
    if mode:
        assert "k_prev 16 bytes" in seen


def _resources(src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", os.path.join(root, "include"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c", os.path.join(root, src),
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    kernels, cur = {}, None
    for line in out.stderr.splitlines():
        m = re.search(r"remark: +(.*?) \[-Rpass", line)
        if not m:
            continue
        text = m.group(1).strip()
        if text.startswith("Function Name:"):
            cur = text.split(":", 1)[1].strip()
            kernels[cur] = {}
        elif cur and ":" in text:
            k, v = text.split(":", 1)
            kernels[cur][k.strip()] = v.strip()
    return kernels


@pytest.mark.parametrize("src", ["verify.hip", "commit.hip", "storeall.hip", "budget.hip", "attention.hip"])
def test_no_kernel_uses_scratch(src):
    """Every kernel keeps its values in registers and LDS: no private segment (scratch memory)
    and no vector-register spills.  Scalar registers that overflow are parked in lanes of
    vector registers, which touches no memory, so those are allowed."""
    kernels = _resources(os.path.join("speculative_decoding_tree_amd", "csrc", src))
    assert kernels
    for name, r in kernels.items():
        assert r.get("ScratchSize [bytes/lane]") == "0", (name, r)
        assert r.get("VGPRs Spill") == "0", (name, r)
        assert r.get("Dynamic Stack") == "False", (name, r)
