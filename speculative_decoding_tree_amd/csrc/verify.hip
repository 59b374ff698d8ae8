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
// gfx950 layout.  One workgroup (4 wave64) owns one (request, v-head) unit.
// Wave w keeps its 128 x 32 column slab of H0 in registers as the B operand
// of v_mfma_f32_16x16x32_bf16, split into bf16 hi + lo parts (q and k are
// exact bf16, so two MFMAs with fp32 accumulation carry ~16 mantissa bits of
// H0).  Lane (n, grp) of the wave loads float2 columns 32w + 2n, 2n+1 of rows
// 32s + 8grp .. +7; the even columns form n-tile 0 and the odd ones n-tile 1,
// so every load instruction reads whole 128-byte row segments.  The K and Q
// rows of the unit are stacked (K rows 0..N-1, Q rows N..2N-1) in LDS as the A
// operand; wave w also multiplies them by K^T for node columns 16w .. 16w+15,
// which gives the masked grams.  The LDS block that held K/Q is reused for
// R and then U.  H0, q/k, v and the per-node scalars are all requested before
// the first barrier; barriers are LDS-only so those loads stay in flight.
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
    union {
        uint16_t kq[2 * NM][D + 8];   // A operand: K rows then Q rows (bf16)
        float ru[NM][D + 4];          // R, then U after the solve
    } u;
    float A[NM][NM + 1];   // beta_t D_tj KK_tj for strict ancestors j
    float P[NM][NM + 1];   // D_tj QK_tj for inclusive ancestors j
    uint64_t anc[NM];
    float gam[NM], beta[NM], gl[NM];
    int par[NM], dep[NM], lvl_nodes[NM], lvl_start[NM + 2];
    int bad, maxdep;
};

template <int NM>
__global__ __launch_bounds__(NT) void verify_kernel(Args a) {
    constexpr int MT = NM / 8;    // max M-tiles of 16 rows over 2N stacked rows
    constexpr int KT = NM / 16;   // max M-tiles that can hold K rows
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

    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if (st == GDN_TREE_S_BAD_OFFSETS) {
        if (h == 0 && tid == 0 && a.status) a.status[b] = st;
        return;
    }
    const int slot = resolve_slot(a, b);
    const int nmt = (2 * N + 15) >> 4;

    // ---- issue every global read of the unit (nodes first, then H0 and v) ----
    int p_mine = -1;
    float g_mine = 0.f, b_mine = 0.f;
    constexpr int KQ_PER_T = (2 * NM * 16 + NT - 1) / NT;   // 16-byte pieces per lane
    uint4 kq_stage[KQ_PER_T];
    float2 hraw[4][8];
    uint32_t vv[KT][4];
    const bool ok = (st == GDN_TREE_S_OK);
    if (ok) {
        if (tid < N) {
            const size_t gi = (size_t)(lo + tid) * a.Hv + h;
            p_mine = a.parent[lo + tid];
            g_mine = a.g[gi];
            b_mine = a.beta[gi];
        }
#pragma unroll
        for (int e = 0; e < KQ_PER_T; ++e) {
            const int idx = tid + e * NT;
            const int r = idx >> 4, c8 = idx & 15;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (r < N)
                val = reinterpret_cast<const uint4 *>(a.k + ((size_t)(lo + r) * a.Hk + hk) * D)[c8];
            else if (r < 2 * N)
                val = reinterpret_cast<const uint4 *>(a.q + ((size_t)(lo + r - N) * a.Hk + hk) * D)[c8];
            kq_stage[e] = val;
        }
        if (slot >= 0) {
            const float *H = a.S0 + ((size_t)slot * a.Hv + h) * D * D + 32 * w + 2 * n;
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    hraw[s][e] = *reinterpret_cast<const float2 *>(H + (32 * s + 8 * grp + e) * D);
        }
#pragma unroll
        for (int tau = 0; tau < KT; ++tau)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tau + 4 * grp + i;
                vv[tau][i] = 0;
                if (r < N)
                    vv[tau][i] = *reinterpret_cast<const uint32_t *>(
                        a.v + ((size_t)(lo + r) * a.Hv + h) * D + 32 * w + 2 * n);
            }
        // parents, gates and K/Q rows into LDS
        if (tid < N) {
            sm.par[tid] = p_mine;
            sm.gl[tid] = g_mine;
            sm.beta[tid] = b_mine;
        }
        if (w == 0) {
            const bool bad = (tid < N) && (p_mine < -1 || p_mine >= tid);
            const unsigned long long any = __ballot(bad);
            if (lane == 0) sm.bad = any != 0ull;
        }
#pragma unroll
        for (int e = 0; e < KQ_PER_T; ++e) {
            const int idx = tid + e * NT;
            const int r = idx >> 4, c8 = idx & 15;
            if (r < 16 * nmt) *reinterpret_cast<uint4 *>(&sm.u.kq[r][c8 * 8]) = kq_stage[e];
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

    // ---- tree pre-pass: ancestry bitsets and depths ----
    if (tid < N) {
        uint64_t m = 0;
        for (int j = tid; j >= 0; j = sm.par[j]) m |= 1ull << j;
        sm.anc[tid] = m;
        sm.dep[tid] = __popcll(m);
        if (h == 0 && a.anc_mask) a.anc_mask[lo + tid] = m;
    }
    lds_barrier();
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

    // ---- B operands: H0 slab (hi, lo) and K^T for node columns 16w.. ----
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
    if (gram) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            bg[s] = *reinterpret_cast<const u32x4 *>(&sm.u.kq[16 * w + n][32 * s + 8 * grp]);
    }

    // ---- one MFMA pass: [K;Q] x [H0 | K^T] ----
    f32x4 acc[MT][2], gacc[MT];
#pragma unroll
    for (int tau = 0; tau < MT; ++tau) {
        acc[tau][0] = acc[tau][1] = gacc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tau < nmt) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 av = *reinterpret_cast<const u32x4 *>(&sm.u.kq[16 * tau + n][32 * s + 8 * grp]);
                acc[tau][0] = mfma(av, bhi[s][0], acc[tau][0]);
                acc[tau][1] = mfma(av, bhi[s][1], acc[tau][1]);
                acc[tau][0] = mfma(av, blo[s][0], acc[tau][0]);
                acc[tau][1] = mfma(av, blo[s][1], acc[tau][1]);
                if (gram) gacc[tau] = mfma(av, bg[s], gacc[tau]);
            }
        }
    }
    lds_barrier();   // K/Q rows are dead from here; ru reuses their space

    // ---- masked coefficient tables from the grams ----
    if (gram) {
        const int j = 16 * w + n;
#pragma unroll
        for (int tau = 0; tau < MT; ++tau) {
            if (tau < nmt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * tau + 4 * grp + i;
                    if (j < N && r < 2 * N) {
                        const bool krow = r < N;
                        const int t = krow ? r : r - N;
                        const uint64_t at = sm.anc[t];
                        if (((at >> j) & 1) && !(krow && j == t)) {
                            uint64_t seg = at & ~sm.anc[j];
                            float sg = 0.f;
                            while (seg) {
                                sg += sm.gl[__builtin_ctzll(seg)];
                                seg &= seg - 1;
                            }
                            const float dtj = expf(sg);
                            if (krow)
                                sm.A[t][j] = sm.beta[t] * dtj * gacc[tau][i];
                            else
                                sm.P[t][j] = dtj * gacc[tau][i];
                        }
                    }
                }
            }
        }
    }
    // ---- right-hand side R_t = beta_t (v_t - gamma_t W_t) ----
#pragma unroll
    for (int tau = 0; tau < KT; ++tau) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * tau + 4 * grp + i;
            if (r < N) {
                const float bt = sm.beta[r], gm = sm.gam[r];
                float2 rr;
                rr.x = bt * (bf16_lo(vv[tau][i]) - gm * acc[tau][0][i]);
                rr.y = bt * (bf16_hi(vv[tau][i]) - gm * acc[tau][1][i]);
                *reinterpret_cast<float2 *>(&sm.u.ru[r][32 * w + 2 * n]) = rr;
            }
        }
    }

    // ---- forward substitution over depth levels ----
    const int maxdep = sm.maxdep;
    for (int L = 2; L <= maxdep; ++L) {
        lds_barrier();
        const int s0 = sm.lvl_start[L], cnt = sm.lvl_start[L + 1] - s0;
        for (int idx = tid; idx < cnt * (D / 2); idx += NT) {
            const int t = sm.lvl_nodes[s0 + (idx >> 6)], c = 2 * (idx & 63);
            uint64_t m = sm.anc[t] & ~(1ull << t);
            float2 acc2 = *reinterpret_cast<const float2 *>(&sm.u.ru[t][c]);
            while (m) {
                const int j = __builtin_ctzll(m);
                const float aj = sm.A[t][j];
                const float2 uj = *reinterpret_cast<const float2 *>(&sm.u.ru[j][c]);
                acc2.x = fmaf(-aj, uj.x, acc2.x);
                acc2.y = fmaf(-aj, uj.y, acc2.y);
                m &= m - 1;
            }
            *reinterpret_cast<float2 *>(&sm.u.ru[t][c]) = acc2;
        }
    }
    lds_barrier();

    // ---- pseudo-values out (coalesced rows) ----
    for (int idx = tid; idx < N * (D / 4); idx += NT) {
        const int t = idx >> 5, c4 = idx & 31;
        reinterpret_cast<float4 *>(a.U + ((size_t)(lo + t) * a.Hv + h) * D)[c4] =
            *reinterpret_cast<const float4 *>(&sm.u.ru[t][4 * c4]);
    }
    // ---- outputs o_t = gamma_t Z_t + sum_j D_tj QK_tj u_j, from the Z tiles ----
#pragma unroll
    for (int tau = 0; tau < MT; ++tau) {
        if (tau < nmt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tau + 4 * grp + i;
                if (r >= N && r < 2 * N) {
                    const int t = r - N;
                    const int c = 32 * w + 2 * n;
                    const float gm = sm.gam[t];
                    float2 o;
                    o.x = gm * acc[tau][0][i];
                    o.y = gm * acc[tau][1][i];
                    uint64_t m = sm.anc[t];
                    while (m) {
                        const int j = __builtin_ctzll(m);
                        const float pj = sm.P[t][j];
                        const float2 uj = *reinterpret_cast<const float2 *>(&sm.u.ru[j][c]);
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
