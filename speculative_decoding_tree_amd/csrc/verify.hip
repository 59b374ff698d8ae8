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
//   [W; Z] = [K; Q] H0,   [KK; QK] = [K; Q] K^T                (one MFMA pass)
//   R_t = beta_t (v_t - gamma_t W_t)
//   u_t = R_t - sum_{j in anc(t)} beta_t D_tj KK_tj u_j           (level by level)
//   o_t = gamma_t Z_t + sum_{j in anc*(t)} D_tj QK_tj u_j
//
// The tree pre-pass (ancestry bitsets, G, depth levels) runs in wave 0 on
// registers with pointer doubling and ballots while the other waves start
// their MFMAs.
//
// gfx950 layout.  One workgroup (4 wave64) owns one (request, v-head) unit.
// Wave w keeps its 128 x 32 column slab of H0 in registers as the B operand
// of v_mfma_f32_16x16x32_bf16, split into bf16 hi + lo parts (q and k are
// exact bf16, so two MFMAs with fp32 accumulation carry ~16 mantissa bits of
// H0).  Lane (n, grp) of the wave loads float2 columns 32w + 2n, 2n+1 of rows
// 32s + 8grp .. +7; the even columns form n-tile 0 and the odd ones n-tile 1,
// so every load instruction reads whole 128-byte row segments.  A operands
// (16-node tiles of K or Q rows) come from L2, fetched one tile ahead, the
// first ones together with H0.  One MFMA pass over
// the tiles gives W = K H0 (turned into R in LDS at once), Z = Q H0 (kept in
// registers until the outputs) and, in wave w, the grams against K^T for node
// columns 16w .. 16w+15, whose ancestor entries are scaled on the spot into a
// coefficient table.  That pass ends with the only workgroup barrier after
// the tree pre-pass: the solve and the outputs are independent per column,
// so each wave finishes its own 32 columns alone (LDS operations of one wave
// complete in order, so one level's writes are seen by the next level).
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace gdn {
namespace {

constexpr int NT = 256;

// Coefficient table T:
//   T[t][q], q < dep(t) - 1 : A = beta_t D_tj (k_t.k_j) for the ancestor j of t at
//                             position q = dep(j) - 1 of t's root-first list (strict
//                             lower triangle; read by the solve)
//   T[j][t], j <= t         : P_tj = D_tj (q_t.k_j) for ancestors j, 0 otherwise
//                             (upper triangle, node-indexed: the A operand of the
//                             output product (P masked) U)
template <int NM>
struct VerifySmem {
    float ru[NM][D + 4];                       // R, then U after the solve
    float T[NM][NM + 4];
    __attribute__((aligned(16))) uint64_t anc[NM];
    __attribute__((aligned(16))) float gam[NM];
    __attribute__((aligned(16))) float beta[NM];
    __attribute__((aligned(16))) float G2[NM];   // log2(e) * path-cumulative log-decay
    __attribute__((aligned(16))) int dep[NM];
    int lvl_nodes[NM], lvl_start[NM + 2];
    int bad, maxdep;
};

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A fragment of a 16-node tile: lane (n, grp) gets row `row`, elements
// 32 s + 8 grp .. +7 for s = 0..3 (16 bytes each); zero past the last node.
// `base` is the same for the whole workgroup and the per-lane part is a
// 32-bit byte offset, so the address needs no 64-bit vector registers.
__device__ __forceinline__ void load_rows(const uint16_t *base, uint32_t row_stride, int row, int nrows,
                                          int grp, u32x4 (&f)[4]) {
    if (row < nrows) {
        const uint32_t off = ((uint32_t)row * row_stride + 8u * grp) * 2u;
        const char *p = reinterpret_cast<const char *>(base) + off;
#pragma unroll
        for (int s = 0; s < 4; ++s) f[s] = *reinterpret_cast<const u32x4 *>(p + 64 * s);
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) f[s] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int NM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3))) void verify_kernel(Args a) {
    constexpr int KT = NM / 16;   // max 16-node tiles
    // Q tiles are fetched one tile ahead where the registers allow it (the
    // 32-node variant would spill; it loads each Q tile after the previous one).
    constexpr bool QPF = NM != 32;
    __shared__ VerifySmem<NM> sm;

    const int n_units = a.B * a.Hv;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int b = unit / a.Hv;
    const int h = unit - b * a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int n = lane & 15, grp = lane >> 4;
    const int c = 32 * w + 2 * n;   // this lane's column pair

    // H0 depends only on (slot, head): its loads go out before the node
    // offsets come back, so the state is in flight during that round trip.
    const int slot = resolve_slot(a, b);
    float2 hraw[4][8];
    if (slot >= 0) {
        const float *H = a.S0 + ((size_t)slot * a.Hv + h) * D * D + 8 * grp * D + c;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                hraw[s][e] = ld_stream2(H + (32 * s + e) * D);
    }
    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if (st == GDN_TREE_S_BAD_OFFSETS) {
        if (h == 0 && tid == 0 && a.status) a.status[b] = st;
        return;
    }
    const uint32_t krow = (uint32_t)a.Hk * D;   // q/k row stride (elements)
    const uint16_t *kbase = a.k + ((size_t)lo * a.Hk + hk) * D;
    const uint16_t *qbase = a.q + ((size_t)lo * a.Hk + hk) * D;
    const uint16_t *vbase = a.v + ((size_t)lo * a.Hv + h) * D;   // + 32-bit per-lane offsets
    const uint32_t vrow = (uint32_t)a.Hv * D;

    // ---- issue the unit's remaining global reads: per-node scalars, v, K, Q ----
    int p_mine = -1;
    float g_mine = 0.f, b_mine = 0.f;
    uint32_t vv[4];   // v of the current K tile's rows (the next tile's come with its A fragments)
    // A fragments of the first K and Q tiles and the K rows of this wave's gram
    // columns are issued with H0; later tiles are fetched one tile ahead.
    const bool gram = 16 * w < N;
    const int jcol = 16 * w + n;   // gram column (node) of this lane
    u32x4 ka[4], qa[4], bg[4];
    if (st == GDN_TREE_S_OK && N > 0) {
        const int tc = min(tid, N - 1);
        const size_t gi = (size_t)(lo + tc) * a.Hv + h;
        p_mine = a.parent[lo + tc];
        g_mine = a.g[gi];
        b_mine = a.beta[gi];
#pragma unroll
        for (int i = 0; i < 4; ++i)   // rows past N read the last row; their R rows are never used
            vv[i] = *reinterpret_cast<const uint32_t *>(vbase + ((uint32_t)min(4 * grp + i, N - 1) * vrow + c));
        load_rows(kbase, krow, jcol, N, grp, bg);
        load_rows(kbase, krow, n, N, grp, ka);
        if (tid < N) sm.beta[tid] = b_mine;
        if (w == 0) {
            const bool bad = (tid < N) && (p_mine < -1 || p_mine >= tid);
            const unsigned long long any = __ballot(bad);
            if (lane == 0) sm.bad = any != 0ull;
        }
        lds_barrier();
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

    // ---- B operands: H0 slab (hi, lo) and K^T for node columns 16w .. 16w+15 ----
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
    lds_barrier();   // ancestry, G, gamma, depths, levels visible

    // ---- one MFMA pass: K tiles -> R, Q tiles -> Z (registers), grams -> T ----
    const int nkt = (N + 15) >> 4;
    const float G2_j = gram && jcol < N ? sm.G2[jcol] : 0.f;
    const int qj = gram && jcol < N ? sm.dep[jcol] - 1 : 0;   // position of node jcol in its descendants' lists
    f32x4 zt[KT][2];
#pragma unroll
    for (int tau = 0; tau < KT; ++tau) {   // K tiles: R rows and A entries
        if (tau < nkt) {
            u32x4 ak[4], nx[4];
            uint32_t vc[4], vn[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ak[s] = ka[s];
                vc[s] = vv[s];
            }
            if (tau + 1 == nkt) load_rows(qbase, krow, n, N, grp, qa);
            if (tau + 1 < KT) {
                load_rows(kbase, krow, 16 * (tau + 1) + n, N, grp, nx);   // zeros past N
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vn[i] = *reinterpret_cast<const uint32_t *>(vbase + ((uint32_t)min(16 * (tau + 1) + 4 * grp + i, N - 1) * vrow + c));
            }
            f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = w0, gk = w0;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                w0 = mfma(ak[s], bhi[s][0], w0);
                w1 = mfma(ak[s], bhi[s][1], w1);
                w0 = mfma(ak[s], blo[s][0], w0);
                w1 = mfma(ak[s], blo[s][1], w1);
                if (gram) gk = mfma(ak[s], bg[s], gk);
            }
            // rows r0 .. r0+3 of this lane (rows past N are scratch rows of ru)
            const int r0 = 16 * tau + 4 * grp;
            const float4 bt4 = *reinterpret_cast<const float4 *>(&sm.beta[r0]);
            const float4 gm4 = *reinterpret_cast<const float4 *>(&sm.gam[r0]);
            const float4 g24 = *reinterpret_cast<const float4 *>(&sm.G2[r0]);
            const float bt[4] = {bt4.x, bt4.y, bt4.z, bt4.w};
            const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
            const float g2[4] = {g24.x, g24.y, g24.z, g24.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + i;
                float2 rr;
                rr.x = bt[i] * (bf16_lo(vc[i]) - gm[i] * w0[i]);
                rr.y = bt[i] * (bf16_hi(vc[i]) - gm[i] * w1[i]);
                *reinterpret_cast<float2 *>(&sm.ru[r][c]) = rr;
                // strict ancestor jcol of r: A = beta_r D_rj (k_r.k_j) at position dep(j)-1
                if (gram && jcol < r && ((sm.anc[r] >> jcol) & 1ull))
                    sm.T[r][qj] = bt[i] * exp2_fast(g2[i] - G2_j) * gk[i];
            }
            if (tau + 1 < KT)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    ka[s] = nx[s];
                    vv[s] = vn[s];
                }
        }
        __builtin_amdgcn_sched_barrier(0);   // one tile's operands live at a time
    }
#pragma unroll
    for (int tau = 0; tau < KT; ++tau) {   // Q tiles: Z kept in registers, P entries
        zt[tau][0] = zt[tau][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tau < nkt) {
            u32x4 aq[4], nx[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) aq[s] = qa[s];
            if (QPF && tau + 1 < KT) load_rows(qbase, krow, 16 * (tau + 1) + n, N, grp, nx);
            f32x4 gq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                zt[tau][0] = mfma(aq[s], bhi[s][0], zt[tau][0]);
                zt[tau][1] = mfma(aq[s], bhi[s][1], zt[tau][1]);
                zt[tau][0] = mfma(aq[s], blo[s][0], zt[tau][0]);
                zt[tau][1] = mfma(aq[s], blo[s][1], zt[tau][1]);
                if (gram) gq = mfma(aq[s], bg[s], gq);
            }
            if (gram) {
                const int r0 = 16 * tau + 4 * grp;
                const float4 g24 = *reinterpret_cast<const float4 *>(&sm.G2[r0]);
                const float g2[4] = {g24.x, g24.y, g24.z, g24.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // P_rj = D_rj (q_r.k_j) for an inclusive ancestor jcol of r, 0 for other j <= r
                    const int r = r0 + i;
                    if (jcol < N && jcol <= r)
                        sm.T[jcol][r] = ((sm.anc[r] >> jcol) & 1ull) ? exp2_fast(g2[i] - G2_j) * gq[i] : 0.f;
                }
            }
            if (tau + 1 < KT) {
                if (QPF) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) qa[s] = nx[s];
                } else {
                    load_rows(qbase, krow, 16 * (tau + 1) + n, N, grp, qa);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();   // R rows and every coefficient visible; from here each wave works alone

    // ---- forward substitution over depth levels, this wave's 32 columns ----
    // Lane (k, p) = (lane >> 4, lane & 15) takes node k of each group of four
    // nodes of the level and the column pair c = 32w + 2p.  U rows go to HBM
    // as soon as their level is done.
    {
        const int kk = lane >> 4;   // == grp
        const int maxdep = sm.maxdep;
        const size_t ustride = (size_t)a.Hv * D;
        float *Ubase = a.U + ((size_t)lo * a.Hv + h) * D + c;
        for (int L = 1; L <= maxdep; ++L) {
            const int s0 = sm.lvl_start[L], cnt = sm.lvl_start[L + 1] - s0;
            for (int g0 = 0; g0 < cnt; g0 += 4) {
                if (g0 + kk < cnt) {
                    const int t = sm.lvl_nodes[s0 + g0 + kk];
                    float2 acc2 = *reinterpret_cast<const float2 *>(&sm.ru[t][c]);
                    uint64_t m = sm.anc[t] & ~(1ull << t);   // the L-1 strict ancestors, root first
                    for (int q = 0; q < L - 1; ++q) {
                        const int j = __builtin_ctzll(m);
                        m &= m - 1;
                        const float aj = sm.T[t][q];
                        const float2 uj = *reinterpret_cast<const float2 *>(&sm.ru[j][c]);
                        acc2.x = fmaf(-aj, uj.x, acc2.x);
                        acc2.y = fmaf(-aj, uj.y, acc2.y);
                    }
                    if (L > 1) *reinterpret_cast<float2 *>(&sm.ru[t][c]) = acc2;
                    st_stream2(Ubase + (size_t)t * ustride, acc2);
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
    {
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
                    if (tau < nkt) {
                        const int t = 16 * tau + n;
                        u32x4 pah, pal;
#pragma unroll
                        for (int pr = 0; pr < 4; ++pr) {
                            const int j0 = 32 * ks + 8 * grp + 2 * pr;
                            const int jr = j0 < NM ? j0 : 0;
                            float p0 = sm.T[jr][t], p1 = sm.T[jr + 1][t];
                            if (j0 > t || j0 >= N) p0 = 0.f;
                            if (j0 + 1 > t || j0 + 1 >= N) p1 = 0.f;
                            uint32_t hh, ll;
                            split_bf16x2(p0, p1, hh, ll);
                            pah[pr] = hh;
                            pal[pr] = ll;
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
    }
}

}  // namespace

hipError_t launch_verify(const Args &a, hipStream_t stream) {
    const dim3 grid(xcd_grid(a.B * a.Hv)), block(NT);
    if (a.max_nodes <= 16)
        verify_kernel<16><<<grid, block, 0, stream>>>(a);
    else if (a.max_nodes <= 32)
        verify_kernel<32><<<grid, block, 0, stream>>>(a);
    else
        verify_kernel<64><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
