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
// (16-node tiles of K or Q rows) come straight from L2.  Pass 1 runs the K
// tiles: W = K H0 becomes R in LDS, and wave w also multiplies K and Q tiles
// by K^T for node columns 16w .. 16w+15 (the grams).  After the solve, pass 2
// runs the Q tiles and turns each Z tile into outputs directly, so only one
// tile of accumulators is ever live.  The grams share one LDS table: A_tj in
// the strict lower triangle, P_tj stored transposed in the upper triangle.
// H0, v and the per-node scalars are all requested before the first barrier;
// barriers are LDS-only so those loads stay in flight.
#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int NT = 256;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier that orders LDS only: outstanding global loads are not
// waited for (HIP's __syncthreads fences global memory as well).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two floats to a packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r;
    r.x = (__bf16)a;
    r.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

// x = hi + lo + O(2^-16 |x|): hi = bf16(x), lo = bf16(x - hi) (x - hi is exact).
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pack_bf16x2(a, b);
    const float ha = __uint_as_float(hi << 16);
    const float hb = __uint_as_float(hi & 0xffff0000u);
    lo = pack_bf16x2(a - ha, b - hb);
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int NM>
struct VerifySmem {
    float ru[NM][D + 4];   // R, then U after the solve
    float T[NM][NM + 1];   // [t][j], j < t: beta_t D_tj KK_tj;  [j][t], j <= t: D_tj QK_tj
    uint64_t anc[NM];
    float gam[NM], beta[NM], G[NM];
    int lvl_nodes[NM], lvl_start[NM + 2];
    int bad, maxdep;
};

// A or B fragment of a 16-node tile: lane (n, grp) gets row `row`, elements
// 32 s + 8 grp .. +7 for s = 0..3 (16 bytes each); zero past the last node.
__device__ __forceinline__ void load_rows(const uint16_t *base, size_t row_stride, int row, int nrows,
                                          int grp, u32x4 (&f)[4]) {
    if (row < nrows) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(base + (size_t)row * row_stride + 8 * grp);
#pragma unroll
        for (int s = 0; s < 4; ++s) f[s] = p[4 * s];
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) f[s] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int NM>
__global__ __launch_bounds__(NT) void verify_kernel(Args a) {
    constexpr int KT = NM / 16;   // max 16-node tiles
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

    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if (st == GDN_TREE_S_BAD_OFFSETS) {
        if (h == 0 && tid == 0 && a.status) a.status[b] = st;
        return;
    }
    const int slot = resolve_slot(a, b);
    const int nkt = (N + 15) >> 4;
    const size_t krow = (size_t)a.Hk * D;            // q/k row stride (elements)
    const uint16_t *kbase = a.k + ((size_t)lo * a.Hk + hk) * D;
    const uint16_t *qbase = a.q + ((size_t)lo * a.Hk + hk) * D;

    // ---- issue the unit's global reads: per-node scalars, H0, v ----
    int p_mine = -1;
    float g_mine = 0.f, b_mine = 0.f;
    float2 hraw[4][8];
    uint32_t vv[KT][4];
    if (st == GDN_TREE_S_OK) {
        if (tid < N) {
            const size_t gi = (size_t)(lo + tid) * a.Hv + h;
            p_mine = a.parent[lo + tid];
            g_mine = a.g[gi];
            b_mine = a.beta[gi];
        }
        if (slot >= 0) {
            const float *H = a.S0 + ((size_t)slot * a.Hv + h) * D * D + 8 * grp * D + c;
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    hraw[s][e] = *reinterpret_cast<const float2 *>(H + (32 * s + e) * D);
        }
#pragma unroll
        for (int tau = 0; tau < KT; ++tau)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tau + 4 * grp + i;
                vv[tau][i] = 0;
                if (r < N)
                    vv[tau][i] = *reinterpret_cast<const uint32_t *>(a.v + ((size_t)(lo + r) * a.Hv + h) * D + c);
            }
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
        if (live) {
            sm.anc[lane] = m;
            sm.G[lane] = G;
            sm.gam[lane] = expf(G);
            sm.lvl_nodes[pos] = lane;
            if (h == 0 && a.anc_mask) a.anc_mask[lo + lane] = m;
        }
    }

    // ---- B operands: H0 slab (hi, lo); K^T for node columns 16w .. 16w+15 ----
    u32x4 bhi[4][2], blo[4][2], bg[4];
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
    const bool gram = 16 * w < N;
    const int jcol = 16 * w + n;   // gram column (node) of this lane
    if (gram) load_rows(kbase, krow, jcol, N, grp, bg);
    lds_barrier();   // ancestry, G, gamma, levels visible

    // ---- pass 1: K tiles -> R rows and raw K.K^T; Q tiles -> raw Q.K^T ----
#pragma unroll
    for (int tau = 0; tau < KT; ++tau) {
        if (tau < nkt) {
            u32x4 af[4];
            load_rows(kbase, krow, 16 * tau + n, N, grp, af);
            f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = w0, gk = w0;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                w0 = mfma(af[s], bhi[s][0], w0);
                w1 = mfma(af[s], bhi[s][1], w1);
                w0 = mfma(af[s], blo[s][0], w0);
                w1 = mfma(af[s], blo[s][1], w1);
                if (gram) gk = mfma(af[s], bg[s], gk);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tau + 4 * grp + i;
                if (r < N) {
                    const float bt = sm.beta[r], gm = sm.gam[r];
                    float2 rr;
                    rr.x = bt * (bf16_lo(vv[tau][i]) - gm * w0[i]);
                    rr.y = bt * (bf16_hi(vv[tau][i]) - gm * w1[i]);
                    *reinterpret_cast<float2 *>(&sm.ru[r][c]) = rr;
                    if (gram && jcol < r) sm.T[r][jcol] = gk[i];
                }
            }
        }
    }
    if (gram) {
#pragma unroll
        for (int tau = 0; tau < KT; ++tau) {
            if (tau < nkt) {
                u32x4 af[4];
                load_rows(qbase, krow, 16 * tau + n, N, grp, af);
                f32x4 gq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) gq = mfma(af[s], bg[s], gq);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tau + 4 * grp + i;
                    if (t < N && jcol <= t) sm.T[jcol][t] = gq[i];
                }
            }
        }
    }
    lds_barrier();

    // ---- decay and beta factors on the ancestor entries only ----
    if (w < 2 && lane < N) {
        const int t = lane;
        const float Gt = sm.G[t];
        uint64_t m = sm.anc[t];
        if (w == 0) {
            const float bt = sm.beta[t];
            m &= ~(1ull << t);
            while (m) {
                const int j = __builtin_ctzll(m);
                sm.T[t][j] *= bt * expf(Gt - sm.G[j]);
                m &= m - 1;
            }
        } else {
            while (m) {
                const int j = __builtin_ctzll(m);
                sm.T[j][t] *= expf(Gt - sm.G[j]);
                m &= m - 1;
            }
        }
    }

    // ---- forward substitution over depth levels ----
    const int maxdep = sm.maxdep;
    for (int L = 2; L <= maxdep; ++L) {
        lds_barrier();
        const int s0 = sm.lvl_start[L], cnt = sm.lvl_start[L + 1] - s0;
        for (int idx = tid; idx < cnt * (D / 2); idx += NT) {
            const int t = sm.lvl_nodes[s0 + (idx >> 6)], cc = 2 * (idx & 63);
            uint64_t m = sm.anc[t] & ~(1ull << t);
            float2 acc2 = *reinterpret_cast<const float2 *>(&sm.ru[t][cc]);
            while (m) {
                const int j = __builtin_ctzll(m);
                const float aj = sm.T[t][j];
                const float2 uj = *reinterpret_cast<const float2 *>(&sm.ru[j][cc]);
                acc2.x = fmaf(-aj, uj.x, acc2.x);
                acc2.y = fmaf(-aj, uj.y, acc2.y);
                m &= m - 1;
            }
            *reinterpret_cast<float2 *>(&sm.ru[t][cc]) = acc2;
        }
    }
    lds_barrier();

    // ---- pseudo-values out (coalesced rows) ----
    for (int idx = tid; idx < N * (D / 4); idx += NT) {
        const int t = idx >> 5, c4 = idx & 31;
        reinterpret_cast<float4 *>(a.U + ((size_t)(lo + t) * a.Hv + h) * D)[c4] =
            *reinterpret_cast<const float4 *>(&sm.ru[t][4 * c4]);
    }
    // ---- pass 2: Q tiles -> Z -> o_t = gamma_t Z_t + sum_j D_tj QK_tj u_j ----
#pragma unroll
    for (int tau = 0; tau < KT; ++tau) {
        if (tau < nkt) {
            u32x4 af[4];
            load_rows(qbase, krow, 16 * tau + n, N, grp, af);
            f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = z0;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                z0 = mfma(af[s], bhi[s][0], z0);
                z1 = mfma(af[s], bhi[s][1], z1);
                z0 = mfma(af[s], blo[s][0], z0);
                z1 = mfma(af[s], blo[s][1], z1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tau + 4 * grp + i;
                if (t < N) {
                    const float gm = sm.gam[t];
                    float2 o;
                    o.x = gm * z0[i];
                    o.y = gm * z1[i];
                    uint64_t m = sm.anc[t];
                    while (m) {
                        const int j = __builtin_ctzll(m);
                        const float pj = sm.T[j][t];
                        const float2 uj = *reinterpret_cast<const float2 *>(&sm.ru[j][c]);
                        o.x = fmaf(pj, uj.x, o.x);
                        o.y = fmaf(pj, uj.y, o.y);
                        m &= m - 1;
                    }
                    *reinterpret_cast<float2 *>(a.out + ((size_t)(lo + t) * a.Hv + h) * D + c) = o;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_verify(const Args &a, hipStream_t stream) {
    const int n_units = a.B * a.Hv;
    const dim3 grid(xcd_grid(n_units)), block(NT);
    if (a.max_nodes <= 16)
        verify_kernel<16><<<grid, block, 0, stream>>>(a);
    else if (a.max_nodes <= 32)
        verify_kernel<32><<<grid, block, 0, stream>>>(a);
    else
        verify_kernel<64><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
