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
//   W = K H0,  Z = Q H0                                  (state products)
//   R_t = beta_t (v_t - gamma_t W_t)
//   u_t = R_t - sum_{j in anc(t)} beta_t D_tj (k_t.k_j) u_j    (level by level)
//   o_t = gamma_t Z_t + sum_{j in anc*(t)} D_tj (q_t.k_j) u_j
//
// One workgroup (256 lanes, 4 wave64) owns one (request, v-head) unit.
#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int NT = 256;

template <int NM>
struct VerifySmem {
    uint16_t K[NM][D];      // key rows of the unit's key head (bf16)
    uint16_t Q[NM][D];      // query rows (bf16)
    float W[NM][D];         // K.H0, then R, then U
    float Z[NM][D];         // Q.H0
    float A[NM][NM + 1];    // beta_t D_tj (k_t.k_j) for strict ancestors j
    float P[NM][NM + 1];    // D_tj (q_t.k_j) for inclusive ancestors j
    uint64_t anc[NM];
    float gam[NM], beta[NM], gl[NM];
    int par[NM], dep[NM];
    int lvl_nodes[NM];
    int lvl_start[NM + 2];
    int bad, maxdep;
};

__device__ __forceinline__ float dot8_bf16(uint4 x, uint4 y, float acc) {
    acc = fmaf(bf16_lo(x.x), bf16_lo(y.x), acc);
    acc = fmaf(bf16_hi(x.x), bf16_hi(y.x), acc);
    acc = fmaf(bf16_lo(x.y), bf16_lo(y.y), acc);
    acc = fmaf(bf16_hi(x.y), bf16_hi(y.y), acc);
    acc = fmaf(bf16_lo(x.z), bf16_lo(y.z), acc);
    acc = fmaf(bf16_hi(x.z), bf16_hi(y.z), acc);
    acc = fmaf(bf16_lo(x.w), bf16_lo(y.w), acc);
    acc = fmaf(bf16_hi(x.w), bf16_hi(y.w), acc);
    return acc;
}

__device__ __forceinline__ float axpy8_bf16(uint4 x, const float *hv, float acc) {
    acc = fmaf(bf16_lo(x.x), hv[0], acc);
    acc = fmaf(bf16_hi(x.x), hv[1], acc);
    acc = fmaf(bf16_lo(x.y), hv[2], acc);
    acc = fmaf(bf16_hi(x.y), hv[3], acc);
    acc = fmaf(bf16_lo(x.z), hv[4], acc);
    acc = fmaf(bf16_hi(x.z), hv[5], acc);
    acc = fmaf(bf16_lo(x.w), hv[6], acc);
    acc = fmaf(bf16_hi(x.w), hv[7], acc);
    return acc;
}

template <int NM>
__global__ __launch_bounds__(NT) void verify_kernel(Args a) {
    __shared__ VerifySmem<NM> sm;
    const int n_units = a.B * a.Hv;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int b = unit / a.Hv;
    const int h = unit - b * a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int tid = threadIdx.x;

    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if (st == GDN_TREE_S_BAD_OFFSETS) {
        if (h == 0 && tid == 0 && a.status) a.status[b] = st;
        return;
    }
    if (st == GDN_TREE_S_OK) {
        if (tid == 0) sm.bad = 0;
        __syncthreads();
        for (int t = tid; t < N; t += NT) {
            const int p = a.parent[lo + t];
            sm.par[t] = p;
            if (p < -1 || p >= t) sm.bad = 1;
        }
        __syncthreads();
        if (sm.bad) st = GDN_TREE_S_BAD_PARENT;
    }
    int slot = -1;
    if (st == GDN_TREE_S_OK) {
        slot = resolve_slot(a, b);
        if (slot < 0) st = GDN_TREE_S_BAD_SLOT;
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

    // ---- tree pre-pass: ancestry bitsets, depths, per-node gate and beta ----
    if (tid < N) {
        const int t = tid;
        uint64_t m = 0;
        for (int j = t; j >= 0; j = sm.par[j]) m |= 1ull << j;
        sm.anc[t] = m;
        sm.dep[t] = __popcll(m);
        const size_t gi = (size_t)(lo + t) * a.Hv + h;
        sm.gl[t] = a.g[gi];
        sm.beta[t] = a.beta[gi];
        if (h == 0 && a.anc_mask) a.anc_mask[lo + t] = m;
    }
    // stage the key head's q and k rows (bf16, 256 B each)
    for (int idx = tid; idx < N * (D / 8); idx += NT) {
        const int t = idx >> 4, c8 = idx & 15;
        const size_t row = ((size_t)(lo + t) * a.Hk + hk) * D;
        *reinterpret_cast<uint4 *>(&sm.K[t][c8 * 8]) = reinterpret_cast<const uint4 *>(a.k + row)[c8];
        *reinterpret_cast<uint4 *>(&sm.Q[t][c8 * 8]) = reinterpret_cast<const uint4 *>(a.q + row)[c8];
    }
    __syncthreads();
    if (tid < N) {
        uint64_t m = sm.anc[tid];
        float G = 0.f;
        while (m) {
            G += sm.gl[__builtin_ctzll(m)];
            m &= m - 1;
        }
        sm.gam[tid] = expf(G);
    }
    if (tid == 0) {  // nodes grouped by depth (counting sort, N <= 64)
        int maxd = 0;
        for (int t = 0; t < N; ++t) maxd = max(maxd, sm.dep[t]);
        int pos = 0;
        for (int d = 1; d <= maxd; ++d) {
            sm.lvl_start[d] = pos;
            for (int t = 0; t < N; ++t)
                if (sm.dep[t] == d) sm.lvl_nodes[pos++] = t;
        }
        sm.lvl_start[maxd + 1] = pos;
        sm.maxdep = maxd;
    }
    // ---- masked grams and decay ratios (ancestor pairs only) ----
    for (int idx = tid; idx < N * N; idx += NT) {
        const int t = idx / N, j = idx - t * N;
        if (!((sm.anc[t] >> j) & 1)) continue;
        float kk = 0.f, qk = 0.f;
#pragma unroll 4
        for (int c8 = 0; c8 < D / 8; ++c8) {
            const uint4 kj = *reinterpret_cast<const uint4 *>(&sm.K[j][c8 * 8]);
            const uint4 kt = *reinterpret_cast<const uint4 *>(&sm.K[t][c8 * 8]);
            const uint4 qt = *reinterpret_cast<const uint4 *>(&sm.Q[t][c8 * 8]);
            kk = dot8_bf16(kt, kj, kk);
            qk = dot8_bf16(qt, kj, qk);
        }
        uint64_t seg = sm.anc[t] & ~sm.anc[j];   // nodes on the path strictly below j
        float s = 0.f;
        while (seg) {
            s += sm.gl[__builtin_ctzll(seg)];
            seg &= seg - 1;
        }
        const float dtj = expf(s);
        sm.P[t][j] = dtj * qk;
        if (j != t) sm.A[t][j] = sm.beta[t] * dtj * kk;
    }

    // ---- state products W = K.H0, Z = Q.H0 (fp32 VALU) ----
    {
        constexpr int RM = NM / 2;
        const int c = tid & (D - 1), rg = tid >> 7;
        float aw[RM], az[RM];
#pragma unroll
        for (int m = 0; m < RM; ++m) aw[m] = az[m] = 0.f;
        const float *H = a.S0 + ((size_t)slot * a.Hv + h) * D * D;
        for (int i0 = 0; i0 < D; i0 += 8) {
            float hv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = H[(i0 + e) * D + c];
#pragma unroll
            for (int m = 0; m < RM; ++m) {
                const int t = rg + 2 * m;
                if (t < N) {
                    aw[m] = axpy8_bf16(*reinterpret_cast<const uint4 *>(&sm.K[t][i0]), hv, aw[m]);
                    az[m] = axpy8_bf16(*reinterpret_cast<const uint4 *>(&sm.Q[t][i0]), hv, az[m]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < RM; ++m) {
            const int t = rg + 2 * m;
            if (t < N) {
                sm.W[t][c] = aw[m];
                sm.Z[t][c] = az[m];
            }
        }
    }
    __syncthreads();

    // ---- right-hand side R_t = beta_t (v_t - gamma_t W_t) ----
    for (int idx = tid; idx < N * D; idx += NT) {
        const int t = idx >> 7, c = idx & (D - 1);
        const float vv = bf16_to_f32(a.v[((size_t)(lo + t) * a.Hv + h) * D + c]);
        sm.W[t][c] = sm.beta[t] * (vv - sm.gam[t] * sm.W[t][c]);
    }
    // ---- forward substitution over depth levels ----
    const int maxdep = sm.maxdep;
    for (int L = 2; L <= maxdep; ++L) {
        __syncthreads();
        const int s0 = sm.lvl_start[L], cnt = sm.lvl_start[L + 1] - s0;
        for (int idx = tid; idx < cnt * D; idx += NT) {
            const int t = sm.lvl_nodes[s0 + (idx >> 7)], c = idx & (D - 1);
            uint64_t m = sm.anc[t] & ~(1ull << t);
            float acc = sm.W[t][c];
            while (m) {
                const int j = __builtin_ctzll(m);
                acc = fmaf(-sm.A[t][j], sm.W[j][c], acc);
                m &= m - 1;
            }
            sm.W[t][c] = acc;
        }
    }
    __syncthreads();

    // ---- outputs and pseudo-values ----
    for (int idx = tid; idx < N * D; idx += NT) {
        const int t = idx >> 7, c = idx & (D - 1);
        const size_t o = ((size_t)(lo + t) * a.Hv + h) * D + c;
        a.U[o] = sm.W[t][c];
        float acc = sm.gam[t] * sm.Z[t][c];
        uint64_t m = sm.anc[t];
        while (m) {
            const int j = __builtin_ctzll(m);
            acc = fmaf(sm.P[t][j], sm.W[j][c], acc);
            m &= m - 1;
        }
        a.out[o] = acc;
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
