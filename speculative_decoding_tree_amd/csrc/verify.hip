// gdn_tree_verify: every draft node's output and pseudo-value from the
// committed state with one ancestor-masked unit-lower-triangular solve.
//
// TreeWY (arXiv 2608.20961), "Method" and "Novelty": nodes are ordered
// parent-before-child, each node's pseudo-value couples only to its
// ancestors, all pseudo-values come from one triangular system, and the
// outputs are read from the same pseudo-values.  Per (request b, v-head h),
// with anc*(t) the inclusive ancestors, G_t = sum of g over anc*(t),
// gamma_t = exp(G_t), D_tj = exp(G_t - G_j) and H0 = S0^T ([d_k][d_v]):
//
//   [W; Z] = [K; Q] H0,   [KK; QK] = [K; Q] K^T                (MFMA)
//   R_t = beta_t (v_t - gamma_t W_t)
//   u_t = R_t - sum_{j in anc(t)} beta_t D_tj KK_tj u_j           (level by level)
//   o_t = gamma_t Z_t + sum_{j in anc*(t)} D_tj QK_tj u_j
//
// The tree pre-pass (ancestry bitsets, G, depth levels) runs in wave 0 on
// registers with pointer doubling and ballots while the state is in flight.
//
// gfx950 layout.  One workgroup (4 wave64) owns one (request, v-head) unit;
// units are dealt to the XCDs by head group (xcd_group_unit), so that every
// XCD gets the same share of every request, whatever the mix of tree sizes.
// Wave w keeps its 128 x 32 column slab of H0 in registers as the B operand
// of v_mfma_f32_16x16x32_bf16, split into bf16 hi + lo parts (q and k are
// exact bf16, so two MFMAs with fp32 accumulation carry ~16 mantissa bits of
// H0).  Lane (n, grp) of the wave loads float2 columns 32w + 2n, 2n+1 of rows
// 32s + 8grp .. +7; the even columns form n-tile 0 and the odd ones n-tile 1,
// so every load instruction reads whole 128-byte row segments.
//
// Loads.  Under full load a global round trip costs microseconds, so a unit
// makes one: after the node offsets, every wave requests its share of the
// unit's Q and K rows (staged in LDS) and its v elements, then its H0 slab;
// wave 0 requests the per-node scalars first.  Loads retire in order, so the
// tree pre-pass waits for the scalars and the staged rows but not for H0.
// The staged rows (bf16, XOR-swizzled 16-byte chunks) occupy the R/U area,
// which holds nothing until R is written: Q rows at its start, K rows at its
// end.  Then, from LDS: the grams against K^T for 16 node columns per wave
// (ancestor entries scaled on the spot into a coefficient table; in units of
// up to 32 nodes the K and the Q products go to different waves), the Q pass
// (Z = Q H0 kept in registers), a barrier (the Q rows are dead),
// and the K pass (W = K H0, turned into R in place; an R tile that covers
// staged K rows is written after a barrier, and it only ever covers rows of
// tiles already read).  After the K pass the solve and the outputs are
// independent per column, so each wave finishes its own 32 columns alone (LDS
// operations of one wave complete in order, so one level's writes are seen
// by the next level).
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace gdn {
namespace {

constexpr int NT = 256;
constexpr int PCHUNK = 16;   // accepted-path rows staged per pass (commit_verify)

// Coefficient table T:
//   T[t][q], q < dep(t) - 1 : A = beta_t D_tj (k_t.k_j) for the ancestor j of t at
//                             position q = dep(j) - 1 of t's root-first list (strict
//                             lower triangle; read by the solve)
//   T[j][t], j <= t         : P_tj = D_tj (q_t.k_j) for ancestors j, 0 otherwise
//                             (upper triangle, node-indexed: the A operand of the
//                             output product (P masked) U), stored as its bf16 hi
//                             and lo parts (hi in the low half of the word), split
//                             once here rather than in every wave that reads it
template <int NM, bool FUSED>
struct VerifySmem {
    // Rows padded by two floats: rows eight apart (the four lane groups of an
    // output fragment read) fall on different banks.
    float ru[NM][D + 2];                       // staged Q and K rows, then R, then U after the solve
    union {
        float T[NM][NM + 2];
        // commit_verify, before the grams: D_aj k_j rows, then u_j rows, of a
        // chunk of the previous tree's accepted path
        float prow[FUSED ? 2 * PCHUNK : 1][D];
    };
    int cpath[FUSED ? 64 : 1];                 // commit_verify: the path, root first
    float ccoef[FUSED ? 64 : 1];               // and its decay coefficients D_aj
    float cgam;
    int cL;
    __attribute__((aligned(16))) uint64_t anc[NM];
    __attribute__((aligned(16))) float gam[NM];
    __attribute__((aligned(16))) float beta[64];   // one per wave-0 lane (clamped copies past N)
    __attribute__((aligned(16))) float G2[NM];   // log2(e) * path-cumulative log-decay
    __attribute__((aligned(16))) int dep[NM];
    int lvl_nodes[NM], lvl_start[NM + 2];
    int bad, maxdep;
};

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Staging rule of the R/U area (bytes, rows of 2D bf16 per staged row): the
// Q rows sit at its start and are dead before any R tile is written; the K
// rows sit at its end, and R tile tau (written after the K pass has read K
// tile tau in every wave) may cover staged K rows of tiles 0 .. tau only.
constexpr bool staging_rule_holds(int nm, int row_bytes) {
    const int ru_bytes = nm * row_bytes, koff = ru_bytes - nm * 2 * D;
    if (koff < nm * 2 * D) return false;   // Q and K rows must not overlap
    for (int tau = 0; tau < nm / 16; ++tau) {
        const int end = (tau + 1) * 16 * row_bytes;   // R tile tau ends here
        if (end > koff && (end - koff + 2 * D - 1) / (2 * D) > 16 * (tau + 1)) return false;
    }
    return true;
}

// Byte offset of 16-byte chunk `chunk` (0..15) of row `row` in a staging
// area of bf16 rows (256 bytes each): chunks are XOR-swizzled by the row so
// that a fragment read (16 rows, one chunk each) hits distinct banks.
__device__ __forceinline__ uint32_t stage_off(int row, int chunk) {
    return (uint32_t)row * (2 * D) + ((uint32_t)(chunk ^ (row & 15)) << 4);
}

// A fragment of a 16-node tile from a staging area: lane (n, grp) gets row
// `row`, elements 32 s + 8 grp .. +7 for s = 0..3 (chunk 4 s + grp).
__device__ __forceinline__ void lds_rows(const char *st, int row, int grp, u32x4 (&f)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) f[s] = *reinterpret_cast<const u32x4 *>(st + stage_off(row, 4 * s + grp));
}

// Occupancy: units of up to 32 nodes fit 128 registers and 23 KiB of LDS, so
// four workgroups share a CU; the 64-node build needs 148 registers and 52 KiB
// and runs three.
//
// MODE 1 (gdn_tree_commit_verify) and 2 (gdn_tree_accept_commit_verify):
// before the verify, the previous tree's accepted path is composed into the
// state while it sits in registers (H' = gamma_a H0 + sum_j D_aj k_j u_j^T,
// in the order and precision of the commit kernel), H' is written to S_out,
// and the verify runs on H'.  Wave 1 derives the path while the state is in
// flight: from the accepted node (MODE 1), or by the greedy walk over the
// previous tree's draft and target tokens (MODE 2).  The path's k and u rows
// are staged in LDS (in the coefficient table's space, which holds nothing
// before the grams).
template <int NM, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NM <= 32 ? 4 : 3))) void verify_kernel(Args a) {
    constexpr bool FUSED = MODE != 0, GREEDY = MODE == 2;
    constexpr int KT = NM / 16;   // max 16-node tiles
    // The unit's Q and K rows are staged in the R/U area, which holds nothing
    // before the K pass writes R: Q rows from its start (dead after the Q
    // pass), K rows at its end.  An R tile covers staged K rows of tiles up to
    // its own only, and is written after a barrier when it covers any.
    constexpr int RU_BYTES = NM * (D + 2) * 4;
    constexpr int KOFF = RU_BYTES - NM * 2 * D;
    static_assert(KOFF % 16 == 0, "staged rows are read 16 bytes at a time");
    static_assert(staging_rule_holds(NM, (D + 2) * 4), "an R tile would overwrite K rows still to be read");
    __shared__ VerifySmem<NM, FUSED> sm;
    char *const stq = reinterpret_cast<char *>(&sm.ru[0][0]);
    char *const stk = stq + KOFF;

    const int unit = xcd_group_unit(blockIdx.x, a.B, a.Hk, a.Hv / a.Hk);
    if (unit < 0) return;
    const int b = unit / a.Hv;
    const int h = unit - b * a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, grp = lane >> 4;
    const int c = 32 * w + 2 * n;   // this lane's column pair

    const int slot = resolve_slot(a, b);
    float2 hraw[4][8];
    const size_t hoff = ((size_t)max(slot, 0) * a.Hv + h) * D * D + 8 * grp * D + c;
    const float *H = a.S0 + hoff;
    auto issue_h0 = [&]() {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                hraw[s][e] = ld_stream2(H + (32 * s + e) * D);
    };
    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if constexpr (!FUSED) {
        if (st == GDN_TREE_S_BAD_OFFSETS) {
            if (h == 0 && tid == 0 && a.status) a.status[b] = st;
            return;
        }
    } else if (st == GDN_TREE_S_BAD_OFFSETS) {
        lo = N = 0;   // the tree's rows are unknown: none is read or written
    }
    const uint32_t krow = (uint32_t)a.Hk * D;   // q/k row stride (elements)
    const uint16_t *kbase = a.k + ((size_t)lo * a.Hk + hk) * D;
    const uint16_t *qbase = a.q + ((size_t)lo * a.Hk + hk) * D;
    const uint16_t *vbase = a.v + ((size_t)lo * a.Hv + h) * D;   // + 32-bit per-lane offsets
    const uint32_t vrow = (uint32_t)a.Hv * D;
    // Grams: wave w takes node columns 16 ct .. 16 ct + 15 against the K rows
    // (A entries) and/or the Q rows (P entries).  Units of more than 32 nodes:
    // each wave both, for ct = w.  Smaller ones would leave waves idle, so the
    // two products go to different waves.
    const int nkt = (N + 15) >> 4;
    int ct = w;
    bool kgram = 16 * w < N, qgram = kgram;
    if (nkt == 1) {
        ct = 0;
        kgram = w == 0;
        qgram = w == 1;
    } else if (nkt == 2) {
        ct = w & 1;
        kgram = w < 2;
        qgram = w >= 2;
    }
    const bool gram = kgram || qgram;
    const int jcol = 16 * ct + n;   // gram column (node) of this lane

    // ---- the unit's remaining global reads: per-node scalars, staged Q/K rows, v ----
    int p_mine = -1;
    float g_mine = 0.f, b_mine = 0.f;
    uint32_t vv[KT][4];   // v rows 16 tau + 4 grp + i, columns c, c + 1 (clamped to the last node)
    u32x4 sq[KT], sk[KT];   // chunk tid & 15 of Q and K row 16 tau + (tid >> 4) (clamped)
    const int srow = tid >> 4, sch = tid & 15;
    auto issue_rest = [&]() {
#pragma unroll
        for (int tau = 0; tau < KT; ++tau)
            if (tau < nkt) {
                const uint32_t off = ((uint32_t)min(16 * tau + srow, N - 1) * krow) * 2u + 16u * sch;
                sq[tau] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(qbase) + off);
                sk[tau] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(kbase) + off);
            }
#pragma unroll
        for (int tau = 0; tau < KT; ++tau)
            if (tau < nkt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vv[tau][i] = *reinterpret_cast<const uint32_t *>(
                        vbase + ((uint32_t)min(16 * tau + 4 * grp + i, N - 1) * vrow + c));
    };
    // commit_verify: the previous tree's offsets, and in wave 1 its parents and
    // gates (lane t = node t, clamped), requested before anything else
    // (greedy: also its draft and target tokens, and the root's target token)
    int cst = GDN_TREE_S_OK, plo = 0, PN = 0, pp = -1, acc_node = -1, root_tok = 0, dtok = 0, ttok = 0;
    float pg = 0.f;
    if constexpr (FUSED) {
        cst = check_offsets_at(a.node_offset_prev, a.T_prev, a.max_nodes_prev, b, plo, PN);
        if constexpr (GREEDY) root_tok = a.root_token[b];
        else acc_node = a.accept_node[b];
        if (w == 1 && cst == GDN_TREE_S_OK && PN > 0) {
            const int tc = min(lane, PN - 1);
            pp = a.parent_prev[plo + tc];
            pg = a.g_prev[(size_t)(plo + tc) * a.Hv + h];
            if constexpr (GREEDY) {
                dtok = a.draft_token[plo + tc];
                ttok = a.target_token[plo + tc];
            }
        }
    }
    const bool tree_ok = st == GDN_TREE_S_OK && N > 0;
    // wave 0 needs its per-node scalars first (tree pre-pass): they and the
    // staged rows go out before its H0 slab, so waiting for them does not
    // wait for the slab
    auto issue_scalars = [&]() {
        const int tc = min(lane, N - 1);
        const size_t gi = (size_t)(lo + tc) * a.Hv + h;
        p_mine = a.parent[lo + tc];
        g_mine = a.g[gi];
        b_mine = a.beta[gi];
    };
    auto check_parents = [&]() {
        sm.beta[lane] = b_mine;
        const bool bad = (lane < N) && (p_mine < -1 || p_mine >= lane);
        const unsigned long long any = __ballot(bad);
        if (lane == 0) sm.bad = any != 0ull;
    };
    if constexpr (!FUSED) {
        if (tree_ok) {
            if (w == 0) {
                issue_scalars();
                issue_rest();
                issue_h0();
                check_parents();
            } else {
                issue_rest();
                issue_h0();
            }
        }
    } else {
        // the state is read whatever the tree holds (the commit needs it);
        // one unconditional issue keeps the loads' waits exact
        if (tree_ok) {
            if (w == 0) issue_scalars();
            issue_rest();
        }
        issue_h0();
        if (tree_ok && w == 0) check_parents();
    }
    if constexpr (FUSED) {
        // ---- the previous tree's accepted path (wave 1), as the commit kernel derives it ----
        if (w == 1) {
            int L = 0, pj = 0, accept = -1;
            if (cst == GDN_TREE_S_OK && __ballot(lane < PN && (pp < -1 || pp >= lane))) cst = GDN_TREE_S_BAD_PARENT;
            if (cst == GDN_TREE_S_OK && slot < 0) cst = GDN_TREE_S_BAD_SLOT;
            if (!GREEDY && cst == GDN_TREE_S_OK && (acc_node < -1 || acc_node >= PN)) cst = GDN_TREE_S_BAD_ACCEPT;
            if (cst == GDN_TREE_S_OK) {
                uint64_t pm = 0;
                if constexpr (GREEDY) {
                    // from the committed root, enter the first child in index order
                    // whose draft token is the target's prediction, until none is
                    int want = root_tok;
                    for (int step = 0; step < PN; ++step) {
                        const uint64_t mk = __ballot(lane < PN && pp == accept && dtok == want);
                        if (!mk) break;
                        accept = __builtin_ctzll(mk);
                        pm |= 1ull << accept;
                        want = __shfl(ttok, accept);
                    }
                } else {
                    pm = ancestors_of(lane, PN, lane < PN ? pp : -1, acc_node);
                }
                L = __popcll(pm);
                pj = path_entry(pm, lane);
            }
            float coef, gam;
            path_decay(lane, L, __shfl(pg, pj), coef, gam);
            if (lane < L) {
                sm.cpath[lane] = pj;
                sm.ccoef[lane] = coef;
            }
            if (h == 0 && a.path_out) {   // one head publishes the root-first path (zero-filled row)
                int32_t *row = a.path_out + (size_t)b * a.max_nodes_prev;
                if (lane < L) row[lane] = pj;
                for (int i = L + lane; i < a.max_nodes_prev; i += 64) row[i] = 0;
            }
            if (lane == 0) {
                sm.cL = L;
                sm.cgam = gam;
                if (h == 0 && a.commit_status) a.commit_status[b] = cst;
                if (h == 0 && a.path_len_out) a.path_len_out[b] = L;
                if (GREEDY && h == 0 && a.accept_out) a.accept_out[b] = accept;
            }
        }
        lds_barrier();
        // staged rows to LDS now, which frees their registers for the commit
        if (tree_ok) {
#pragma unroll
            for (int tau = 0; tau < KT; ++tau)
                if (tau < nkt) {
                    const int row = 16 * tau + srow;
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4 *>(stq + stage_off(row, sch)) = row < N ? sq[tau] : z;
                    *reinterpret_cast<u32x4 *>(stk + stage_off(row, sch)) = row < N ? sk[tau] : z;
                }
        }
        // ---- commit: H' = gamma_a H0 + sum_j D_aj k_j u_j^T on this lane's 64 elements ----
        const int L = sm.cL;
        if (L > 0) {   // a valid path (L = 0 on every error)
            const float gam = sm.cgam;
            const int jr = tid >> 4, e0 = 8 * (tid & 15);   // staging: path row jr, elements e0 .. e0 + 7
            for (int j0 = 0; j0 < L; j0 += PCHUNK) {
                const int nj = min(PCHUNK, L - j0);
                if (j0 > 0) lds_barrier();   // every wave has read the previous chunk
                const int q = j0 + min(jr, nj - 1);
                const int t = sm.cpath[q];
                const u32x4 kr = *reinterpret_cast<const u32x4 *>(a.k_prev + ((size_t)(plo + t) * a.Hk + hk) * D + e0);
                const float *up = a.U_prev + ((size_t)(plo + t) * a.Hv + h) * D + e0;
                const float4 u0 = *reinterpret_cast<const float4 *>(up);
                const float4 u1 = *reinterpret_cast<const float4 *>(up + 4);
                const float cf = sm.ccoef[q];
                if (j0 == 0) {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int e = 0; e < 8; ++e) hraw[s][e] = make_float2(gam * hraw[s][e].x, gam * hraw[s][e].y);
                }
                float4 k0, k1;
                k0.x = cf * bf16_lo(kr[0]);
                k0.y = cf * bf16_hi(kr[0]);
                k0.z = cf * bf16_lo(kr[1]);
                k0.w = cf * bf16_hi(kr[1]);
                k1.x = cf * bf16_lo(kr[2]);
                k1.y = cf * bf16_hi(kr[2]);
                k1.z = cf * bf16_lo(kr[3]);
                k1.w = cf * bf16_hi(kr[3]);
                *reinterpret_cast<float4 *>(&sm.prow[jr][e0]) = k0;
                *reinterpret_cast<float4 *>(&sm.prow[jr][e0 + 4]) = k1;
                *reinterpret_cast<float4 *>(&sm.prow[PCHUNK + jr][e0]) = u0;
                *reinterpret_cast<float4 *>(&sm.prow[PCHUNK + jr][e0 + 4]) = u1;
                lds_barrier();
                for (int jj = 0; jj < nj; ++jj) {
                    const float2 u = *reinterpret_cast<const float2 *>(&sm.prow[PCHUNK + jj][c]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const float4 ka = *reinterpret_cast<const float4 *>(&sm.prow[jj][32 * s + 8 * grp]);
                        const float4 kb = *reinterpret_cast<const float4 *>(&sm.prow[jj][32 * s + 8 * grp + 4]);
                        const float kc[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            hraw[s][e].x = fmaf(kc[e], u.x, hraw[s][e].x);
                            hraw[s][e].y = fmaf(kc[e], u.y, hraw[s][e].y);
                        }
                    }
                }
            }
        }
        if (slot >= 0 && (L > 0 || a.S_out != a.S0)) {
            float *Ho = a.S_out + hoff;
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) st_stream2(Ho + (32 * s + e) * D, hraw[s][e]);
        }
    } else if (tree_ok) {
        lds_barrier();
    }
    if (tree_ok) {
        if (sm.bad) st = GDN_TREE_S_BAD_PARENT;
        else if (slot < 0) st = GDN_TREE_S_BAD_SLOT;
    }
    if (st != GDN_TREE_S_OK) {
        const float qnan = __int_as_float(0x7fc00000);
        for (int idx = tid; idx < N * D; idx += NT) {
            const size_t o = ((size_t)(lo + (idx >> 7)) * a.Hv + h) * D + (idx & (D - 1));
            a.out[o] = qnan;
            a.U[o] = qnan;
        }
        if (h == 0) {
            if (a.anc_mask)
                for (int t = tid; t < N; t += NT) a.anc_mask[lo + t] = 0;
            if (tid == 0 && a.status) a.status[b] = st;
        }
        return;
    }
    if (h == 0 && tid == 0 && a.status) a.status[b] = GDN_TREE_S_OK;
    if (N == 0) return;

    // ---- tree pre-pass in wave 0, lane t = node t, registers only ----
    // Pointer doubling: m is the set of nodes from t up to (excluding) jp and
    // G the sum of their gates; each round joins the segment above, so
    // ceil(log2(depth)) + 1 rounds give the inclusive ancestor set and the
    // path-cumulative log-decay G_t.
    if (w == 0) {
        const bool live = lane < N;
        int jp = live ? p_mine : -1;
        uint64_t m = live ? (1ull << lane) : 0ull;
        float G = live ? g_mine : 0.f;
        while (__ballot(jp >= 0)) {
            const int src = jp >= 0 ? jp : lane;
            const uint64_t m_up = __shfl(m, src);
            const float G_up = __shfl(G, src);
            const int jp_up = __shfl(jp, src);
            if (jp >= 0) {
                m |= m_up;
                G += G_up;
                jp = jp_up;
            }
        }
        const int dep = live ? __popcll(m) : 0;
        int maxd = dep;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) maxd = max(maxd, __shfl_xor(maxd, off));
        int base = 0, pos = 0;
        for (int d = 1; d <= maxd; ++d) {   // nodes grouped by depth, index order inside
            const uint64_t mk = __ballot(dep == d);
            if (dep == d) pos = base + __popcll(mk & ((1ull << lane) - 1ull));
            if (lane == 0) sm.lvl_start[d] = base;
            base += __popcll(mk);
        }
        if (lane == 0) {
            sm.lvl_start[maxd + 1] = base;
            sm.maxdep = maxd;
        }
        if (lane < NM) {   // rows past N get empty ancestry so no coefficient is written for them
            const float G2 = G * LOG2E;
            sm.anc[lane] = m;
            sm.G2[lane] = G2;
            sm.gam[lane] = exp2_fast(G2);
            sm.dep[lane] = dep;
        }
        if (live) {
            sm.lvl_nodes[pos] = lane;
            if (h == 0 && a.anc_mask) a.anc_mask[lo + lane] = m;
        }
    }

    // ---- B operand: H0 slab (hi, lo); staged rows to LDS (zeros past N) ----
    u32x4 bhi[4][2], blo[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            uint32_t h0, l0, h1, l1;
            split_bf16x2(hraw[s][2 * pr].x, hraw[s][2 * pr + 1].x, h0, l0);
            split_bf16x2(hraw[s][2 * pr].y, hraw[s][2 * pr + 1].y, h1, l1);
            bhi[s][0][pr] = h0;
            blo[s][0][pr] = l0;
            bhi[s][1][pr] = h1;
            blo[s][1][pr] = l1;
        }
    }
    if constexpr (!FUSED) {
#pragma unroll
        for (int tau = 0; tau < KT; ++tau)
            if (tau < nkt) {
                const int row = 16 * tau + srow;
                const u32x4 z = {0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4 *>(stq + stage_off(row, sch)) = row < N ? sq[tau] : z;
                *reinterpret_cast<u32x4 *>(stk + stage_off(row, sch)) = row < N ? sk[tau] : z;
            }
    }
    lds_barrier();   // ancestry, G, gamma, depths, levels and the staged rows visible

    // ---- grams against K^T for node columns 16 ct .. 16 ct + 15 (ancestor entries only) ----
    const float G2_j = gram && jcol < N ? sm.G2[jcol] : 0.f;
    const int qj = gram && jcol < N ? sm.dep[jcol] - 1 : 0;   // position of node jcol in its descendants' lists
    if (gram) {
        u32x4 bg[4];
        lds_rows(stk, jcol, grp, bg);   // jcol < 16 nkt: staged (zeros past N)
#pragma unroll
        for (int tau = 0; tau < KT; ++tau) {
            if (tau < nkt) {
                const int r0 = 16 * tau + 4 * grp;
                const float4 g24 = *reinterpret_cast<const float4 *>(&sm.G2[r0]);
                const float g2[4] = {g24.x, g24.y, g24.z, g24.w};
                if (kgram) {   // A = beta_r D_rj (k_r.k_j) for strict ancestors j
                    u32x4 ak[4];
                    lds_rows(stk, 16 * tau + n, grp, ak);
                    f32x4 gk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) gk = mfma(ak[s], bg[s], gk);
                    const float4 bt4 = *reinterpret_cast<const float4 *>(&sm.beta[r0]);
                    const float bt[4] = {bt4.x, bt4.y, bt4.z, bt4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = r0 + i;
                        if (jcol < r && ((sm.anc[r] >> jcol) & 1ull))
                            sm.T[r][qj] = bt[i] * exp2_fast(g2[i] - G2_j) * gk[i];
                    }
                }
                if (qgram) {   // P_rj = D_rj (q_r.k_j) for an inclusive ancestor jcol of r, 0 for other j <= r
                    u32x4 aq[4];
                    lds_rows(stq, 16 * tau + n, grp, aq);
                    f32x4 gq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) gq = mfma(aq[s], bg[s], gq);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = r0 + i;
                        if (jcol < N && jcol <= r) {   // stored split: bf16 hi in the low half, lo in the high half
                            const float pv = ((sm.anc[r] >> jcol) & 1ull) ? exp2_fast(g2[i] - G2_j) * gq[i] : 0.f;
                            uint32_t ph, pl;
                            split_bf16x2(pv, 0.f, ph, pl);
                            sm.T[jcol][r] = __uint_as_float((ph & 0xffffu) | (pl << 16));
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- Q pass: Z = Q H0 kept in registers ----
    f32x4 zt[KT][2];
#pragma unroll
    for (int tau = 0; tau < KT; ++tau) {
        zt[tau][0] = zt[tau][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tau < nkt) {
            u32x4 aq[4];
            lds_rows(stq, 16 * tau + n, grp, aq);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                zt[tau][0] = mfma(aq[s], bhi[s][0], zt[tau][0]);
                zt[tau][1] = mfma(aq[s], bhi[s][1], zt[tau][1]);
                zt[tau][0] = mfma(aq[s], blo[s][0], zt[tau][0]);
                zt[tau][1] = mfma(aq[s], blo[s][1], zt[tau][1]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();   // every wave is done with the staged Q rows: R rows may take their place

    // ---- K pass: W = K H0, turned into R in LDS ----
#pragma unroll
    for (int tau = 0; tau < KT; ++tau) {
        if (tau < nkt) {
            u32x4 ak[4];
            lds_rows(stk, 16 * tau + n, grp, ak);
            f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = w0;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                w0 = mfma(ak[s], bhi[s][0], w0);
                w1 = mfma(ak[s], bhi[s][1], w1);
                w0 = mfma(ak[s], blo[s][0], w0);
                w1 = mfma(ak[s], blo[s][1], w1);
            }
            // this tile's R rows cover staged K rows of tiles <= tau: all waves read them first
            if ((tau + 1) * 16 * (D + 2) * 4 > KOFF) lds_barrier();
            // rows r0 .. r0+3 of this lane (rows past N are scratch rows of ru)
            const int r0 = 16 * tau + 4 * grp;
            const float4 bt4 = *reinterpret_cast<const float4 *>(&sm.beta[r0]);
            const float4 gm4 = *reinterpret_cast<const float4 *>(&sm.gam[r0]);
            const float bt[4] = {bt4.x, bt4.y, bt4.z, bt4.w};
            const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + i;
                float2 rr;
                rr.x = bt[i] * (bf16_lo(vv[tau][i]) - gm[i] * w0[i]);
                rr.y = bt[i] * (bf16_hi(vv[tau][i]) - gm[i] * w1[i]);
                *reinterpret_cast<float2 *>(&sm.ru[r][c]) = rr;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();   // R rows and every coefficient visible; from here each wave works alone

    // ---- forward substitution over depth levels, this wave's 32 columns ----
    // Lane (k, p) = (lane >> 3, lane & 7) takes node k of each group of eight
    // nodes of the level and the column quad 32w + 4p.  U rows go to HBM as
    // soon as their level is done.  usum is a running sum of the lane's
    // pseudo-values: it is non-finite when one of them is (or, harmlessly, when
    // the sum overflows), which sends the wave to the output product that keeps
    // non-finite values inside their subtree.
    float usum = 0.f;
    {
        const int kk = lane >> 3, c4 = 32 * w + 4 * (lane & 7);
        const int maxdep = sm.maxdep;
        const size_t ustride = (size_t)a.Hv * D;
        float *Ubase = a.U + ((size_t)lo * a.Hv + h) * D + c4;
        for (int L = 1; L <= maxdep; ++L) {
            const int s0 = sm.lvl_start[L], cnt = sm.lvl_start[L + 1] - s0;
            for (int g0 = 0; g0 < cnt; g0 += 8) {
                if (g0 + kk < cnt) {
                    const int t = sm.lvl_nodes[s0 + g0 + kk];
                    // ru rows are 8-byte aligned (two floats of padding): float2 pairs
                    float2 a0 = *reinterpret_cast<const float2 *>(&sm.ru[t][c4]);
                    float2 a1 = *reinterpret_cast<const float2 *>(&sm.ru[t][c4 + 2]);
                    uint64_t m = sm.anc[t] & ~(1ull << t);   // the L-1 strict ancestors, root first
                    for (int q = 0; q < L - 1; ++q) {
                        const int j = __builtin_ctzll(m);
                        m &= m - 1;
                        const float aj = sm.T[t][q];
                        const float2 u0 = *reinterpret_cast<const float2 *>(&sm.ru[j][c4]);
                        const float2 u1 = *reinterpret_cast<const float2 *>(&sm.ru[j][c4 + 2]);
                        a0.x = fmaf(-aj, u0.x, a0.x);
                        a0.y = fmaf(-aj, u0.y, a0.y);
                        a1.x = fmaf(-aj, u1.x, a1.x);
                        a1.y = fmaf(-aj, u1.y, a1.y);
                    }
                    if (L > 1) {
                        *reinterpret_cast<float2 *>(&sm.ru[t][c4]) = a0;
                        *reinterpret_cast<float2 *>(&sm.ru[t][c4 + 2]) = a1;
                    }
                    st_stream4(reinterpret_cast<float4 *>(Ubase + (size_t)t * ustride), make_float4(a0.x, a0.y, a1.x, a1.y));
                    usum += (a0.x + a0.y) + (a1.x + a1.y);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }

    // ---- outputs O = diag(gamma) Z + (P masked) U on MFMA ----
    // A operand: P rows t = 16 tau + n, elements j = 32 ks + 8 grp + e (from the
    // transposed table; j > t, j >= N are 0 by select).  B operand: U rows j,
    // this wave's columns (rows j >= N are 0 by select).  Both are split into
    // bf16 hi + lo and combined as hi.hi + hi.lo + lo.hi (~16 mantissa bits).
    //
    // A non-ancestor's pseudo-value still meets its zero in P inside the
    // product, so a non-finite entry (from a NaN or Inf in that node's g, beta
    // or v) would reach every row of the tile as 0 * Inf.  A branch reads only
    // its ancestors (TreeWY, "Method"), so such entries must stay in their
    // subtree: when the wave holds one (rare: see usum), the product runs with
    // non-finite U entries replaced by 0 (select), and afterwards every output
    // whose inclusive ancestors carry a non-finite pseudo-value in its column
    // is set to NaN.  Each value row of the state evolves on its own under the
    // gated delta rule, so this is exactly where sequential decode turns
    // non-finite.  Finite inputs take the plain product: same bits as before.
    auto output_product = [&](auto sanitize) {
        constexpr bool SAN = decltype(sanitize)::value;
        const int nks = (N + 31) >> 5;
#pragma unroll
        for (int tau = 0; tau < KT; ++tau) {
            if (tau < nkt) {
                const int r0 = 16 * tau + 4 * grp;
                const float4 gm4 = *reinterpret_cast<const float4 *>(&sm.gam[r0]);
                const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    zt[tau][0][i] *= gm[i];
                    zt[tau][1][i] *= gm[i];
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < (NM + 31) / 32; ++ks) {
            if (ks < nks) {
                // B fragments for this K step: U rows 32 ks + 8 grp + e, columns c (n-tile 0), c+1 (n-tile 1)
                u32x4 ubh[2], ubl[2];
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const int j0 = 32 * ks + 8 * grp + 2 * pr;
                    const int jr = j0 < NM ? j0 : 0;   // rows past the table (NM = 16) are read in range, then zeroed
                    float2 u0 = *reinterpret_cast<const float2 *>(&sm.ru[jr][c]);
                    float2 u1 = *reinterpret_cast<const float2 *>(&sm.ru[jr + 1][c]);
                    if (j0 >= N) u0 = make_float2(0.f, 0.f);
                    if (j0 + 1 >= N) u1 = make_float2(0.f, 0.f);
                    if constexpr (SAN) {
                        u0.x = __builtin_isfinite(u0.x) ? u0.x : 0.f;
                        u0.y = __builtin_isfinite(u0.y) ? u0.y : 0.f;
                        u1.x = __builtin_isfinite(u1.x) ? u1.x : 0.f;
                        u1.y = __builtin_isfinite(u1.y) ? u1.y : 0.f;
                    }
                    uint32_t h0, l0, h1, l1;
                    split_bf16x2(u0.x, u1.x, h0, l0);
                    split_bf16x2(u0.y, u1.y, h1, l1);
                    ubh[0][pr] = h0;
                    ubl[0][pr] = l0;
                    ubh[1][pr] = h1;
                    ubl[1][pr] = l1;
                }
#pragma unroll
                for (int tau = 0; tau < KT; ++tau) {
                    if (tau < nkt && 32 * ks <= 16 * tau + 15) {   // blocks with every j > t are zero
                        const int t = 16 * tau + n;
                        u32x4 pah, pal;
#pragma unroll
                        for (int pr = 0; pr < 4; ++pr) {
                            const int j0 = 32 * ks + 8 * grp + 2 * pr;
                            const int jr = j0 < NM ? j0 : 0;
                            // entries are stored split (hi | lo << 16); j > t holds A, j >= N nothing
                            uint32_t w0 = __float_as_uint(sm.T[jr][t]), w1 = __float_as_uint(sm.T[jr + 1][t]);
                            if (j0 > t || j0 >= N) w0 = 0u;
                            if (j0 + 1 > t || j0 + 1 >= N) w1 = 0u;
                            pah[pr] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);   // hi(j0) | hi(j0 + 1) << 16
                            pal[pr] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);   // lo(j0) | lo(j0 + 1) << 16
                        }
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) {
                            zt[tau][jj] = mfma(pah, ubh[jj], zt[tau][jj]);
                            zt[tau][jj] = mfma(pah, ubl[jj], zt[tau][jj]);
                            zt[tau][jj] = mfma(pal, ubh[jj], zt[tau][jj]);
                        }
                    }
                }
            }
        }
        if constexpr (SAN) {
            // output (r, column) turns NaN when an inclusive ancestor of r has a
            // non-finite pseudo-value in that column (LDS still holds U)
            const float qnan = __int_as_float(0x7fc00000);
#pragma unroll
            for (int tau = 0; tau < KT; ++tau)
                if (tau < nkt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 16 * tau + 4 * grp + i;
                        if (r >= N) continue;
                        bool bad0 = false, bad1 = false;
                        for (uint64_t m = sm.anc[r]; m; m &= m - 1) {
                            const float2 uj = *reinterpret_cast<const float2 *>(&sm.ru[__builtin_ctzll(m)][c]);
                            bad0 = bad0 || !__builtin_isfinite(uj.x);
                            bad1 = bad1 || !__builtin_isfinite(uj.y);
                        }
                        if (bad0) zt[tau][0][i] = qnan;
                        if (bad1) zt[tau][1][i] = qnan;
                    }
        }
        const size_t ostride = (size_t)a.Hv * D;
        float *Obase = a.out + ((size_t)lo * a.Hv + h) * D + c;
#pragma unroll
        for (int tau = 0; tau < KT; ++tau)
            if (tau < nkt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * tau + 4 * grp + i;
                    if (r < N) st_stream2(Obase + (size_t)r * ostride, make_float2(zt[tau][0][i], zt[tau][1][i]));
                }
    };
    if (__ballot(!__builtin_isfinite(usum)))
        output_product(std::true_type{});
    else
        output_product(std::false_type{});
}

template <int MODE>
hipError_t launch_verify_impl(const Args &a, hipStream_t stream) {
    const dim3 grid(xcd_group_grid(a.B, a.Hk, a.Hv / a.Hk)), block(NT);
    if (a.max_nodes <= 16)
        verify_kernel<16, MODE><<<grid, block, 0, stream>>>(a);
    else if (a.max_nodes <= 32)
        verify_kernel<32, MODE><<<grid, block, 0, stream>>>(a);
    else
        verify_kernel<64, MODE><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const Args &a, hipStream_t stream) { return launch_verify_impl<0>(a, stream); }

hipError_t launch_commit_verify(const Args &a, hipStream_t stream) { return launch_verify_impl<1>(a, stream); }

hipError_t launch_accept_commit_verify(const Args &a, hipStream_t stream) {
    return launch_verify_impl<2>(a, stream);
}

}  // namespace gdn
