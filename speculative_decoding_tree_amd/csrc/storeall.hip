// The snapshot-per-node ("storeall") comparison scheme.
//
// TreeWY (arXiv 2608.20961), "Prior work": vLLM's default keeps the committed
// state and the state of every candidate position, then selects the accepted
// one; a tree needs one state per node.  verify walks each request's nodes in
// parent-before-child order with the sequential gated delta rule and writes
// every node's full state; commit copies the accepted node's state.
#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int NT = 256;

// Under the gated delta rule each value column c of the state (column c of
// H = S^T) evolves on its own: u_c = beta (v_c - alpha (S k)_c) and
// H[i][c] <- alpha H[i][c] + k_i u_c.  So each wave owns 32 columns of every
// state of the unit and walks the whole tree without waiting for the others:
// lane (quad, rg) = (lane >> 3, lane & 7) holds columns 32w + 4 quad .. +3 of
// rows rg + 8 i (i = 0..15) in registers.  The column sums (S_p k)_c and
// (S_p q)_c are reduced over the eight row groups by shuffles; the output is
// o = S_t q = alpha (S_p q) + u (k.q).  Each node's state is written with
// 16-byte plain stores (eight lanes cover one 128-byte row segment).  The
// registers hold one state at a time, so a node whose parent's state is not
// the one held reads it back from memory; the visiting order keeps that rare
// (see the walk below).  A lane re-reads only states it wrote itself, so
// program order makes them visible.
// Rows of bf16 (256 bytes) into LDS by direct global-to-LDS loads: one wave
// instruction moves four rows (lane l: row 4 j + l / 16, 16-byte chunk l % 16,
// written at base + 16 l).  Rows past n read row n - 1 (their LDS rows are
// never used).  `rows` gives the global address of a row.
template <typename RowAddr>
__device__ __forceinline__ void stage_rows(uint16_t (*dst)[D], int n, int w, int lane, RowAddr rows) {
    for (int j = w; 4 * j < n; j += NT / 64) {
        const int row = min(4 * j + (lane >> 4), n - 1);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(rows(row)) + (lane & 15),
                                         (__attribute__((address_space(3))) void *)&dst[4 * j][0], 16, 0, 0);
    }
}

template <int NM>
__global__ __launch_bounds__(NT) void verify_storeall_kernel(Args a) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[NM][D];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[NM][D];
    __shared__ __attribute__((aligned(16))) uint16_t sV[NM][D];
    __shared__ float sG[NM], sB[NM];
    __shared__ int s_order[NM];   // the visiting order: depth-first, leaf children first
    __shared__ int s_par[NM];
    __shared__ uint64_t s_leaf;   // nodes without children
    __shared__ int s_bad;

    const int n_units = a.B * a.Hv;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int b = unit / a.Hv;
    const int h = unit - b * a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;

    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if (st == GDN_TREE_S_BAD_OFFSETS) {
        if (h == 0 && tid == 0 && a.status) a.status[b] = st;
        return;
    }
    const int slot = resolve_slot(a, b);
    const bool run = st == GDN_TREE_S_OK && N > 0 && slot >= 0;
    // Every load of the unit goes out before the one wait: the parents (wave
    // 0), the gates and betas (wave 1), the k, q and v rows (straight to LDS)
    // and the state slab (registers).
    int p_mine = -1;
    float gb = 0.f;
    if (st == GDN_TREE_S_OK && N > 0) {
        if (w == 0) p_mine = a.parent[lo + min(lane, N - 1)];
    }
    const int rg = lane & 7, c = 32 * w + 4 * (lane >> 3);   // rows rg + 8 i, columns c .. c + 3
    const size_t state_elems = (size_t)D * D;
    const float *H0 = a.S0 + ((size_t)max(slot, 0) * a.Hv + h) * state_elems;
    float4 hr[16];
    if (run) {
        if (w == 1) {   // lanes 0..63: the gate, then lanes 64..127 of the pair: beta
            const size_t gi = (size_t)(lo + min(lane, N - 1)) * a.Hv + h;
            gb = a.g[gi];
        } else if (w == 2) {
            const size_t gi = (size_t)(lo + min(lane, N - 1)) * a.Hv + h;
            gb = a.beta[gi];
        }
        stage_rows(sK, N, w, lane, [&](int t) { return a.k + ((size_t)(lo + t) * a.Hk + hk) * D; });
        stage_rows(sQ, N, w, lane, [&](int t) { return a.q + ((size_t)(lo + t) * a.Hk + hk) * D; });
        stage_rows(sV, N, w, lane, [&](int t) { return a.v + ((size_t)(lo + t) * a.Hv + h) * D; });
#pragma unroll
        for (int i = 0; i < 16; ++i) hr[i] = *reinterpret_cast<const float4 *>(H0 + (rg + 8 * i) * D + c);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the direct LDS loads land before the barrier
    if (run && lane < N) {
        if (w == 1) sG[lane] = gb;
        else if (w == 2) sB[lane] = gb;
    }
    if (st == GDN_TREE_S_OK && N > 0 && w == 0) {
        // parent check, then the visiting order (one walk on children masks
        // held one per lane): depth-first, and among the children of a node
        // the leaves first.  A leaf's state is formed from its parent's state
        // without replacing it in registers, so the parent's state is read
        // back only before its second and later children that have children
        // of their own.
        const bool live = lane < N;
        const int p = live ? p_mine : -1;
        const bool bad = __ballot(live && (p < -1 || p >= lane)) != 0ull;
        uint64_t leaf = 0;
        if (!bad && slot >= 0) {
            uint64_t kids = 0;
            for (int q = 0; q < N; ++q) {
                const uint64_t m = __ballot(live && p == q);
                if (lane == q) kids = m;
            }
            leaf = __ballot(live && kids == 0ull);
            const uint64_t roots = __ballot(live && p == -1);
            uint64_t done = 0;
            int cur = -1;   // the node whose children are being visited (-1: the roots)
            for (int k = 0; k < N; ++k) {
                uint64_t avail;
                for (;;) {
                    const uint32_t klo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kids, max(cur, 0));
                    const uint32_t khi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(kids >> 32), max(cur, 0));
                    avail = (cur < 0 ? roots : ((uint64_t)khi << 32 | klo)) & ~done;
                    if (avail || cur < 0) break;
                    cur = __builtin_amdgcn_readlane(p, cur);
                }
                const uint64_t leaves = avail & leaf;
                const int nxt = __builtin_ctzll(leaves ? leaves : avail);
                done |= 1ull << nxt;
                if (lane == 0) s_order[k] = nxt;
                if (!((leaf >> nxt) & 1ull)) cur = nxt;   // descend; after a leaf the same node's children go on
            }
        }
        if (lane < N) s_par[lane] = p;
        if (lane == 0) {
            s_bad = bad;
            s_leaf = leaf;
        }
    }
    __syncthreads();
    if (st == GDN_TREE_S_OK && N > 0 && s_bad) st = GDN_TREE_S_BAD_PARENT;
    if (st == GDN_TREE_S_OK && slot < 0) st = GDN_TREE_S_BAD_SLOT;
    if (h == 0 && tid == 0 && a.status) a.status[b] = st;
    if (st != GDN_TREE_S_OK) {
        const float qnan = __int_as_float(0x7fc00000);
        for (int idx = tid; idx < N * D; idx += NT)
            a.out[((size_t)(lo + (idx >> 7)) * a.Hv + h) * D + (idx & (D - 1))] = qnan;
        return;
    }
    if (N == 0) return;

    // No global load in the walk but a parent's state where the walk backs up
    // (the vector-memory counter retires loads and stores in order, so such a
    // load waits for the stores before it).
    int held = -1;   // node whose state sits in hr (-1 = S0)
    const uint64_t leaf = s_leaf;
    for (int k = 0; k < N; ++k) {
        const int t = s_order[k];
        const int p = s_par[t];
        if (p != held) {
            const float *src = p < 0 ? H0 : a.node_state + ((size_t)(lo + p) * a.Hv + h) * state_elems;
#pragma unroll
            for (int i = 0; i < 16; ++i) hr[i] = *reinterpret_cast<const float4 *>(src + (rg + 8 * i) * D + c);
        }
        const size_t gi = (size_t)(lo + t) * a.Hv + h;
        const float alpha = expf(sG[t]);
        const float beta = sB[t];
        const uint2 vr = *reinterpret_cast<const uint2 *>(&sV[t][c]);
        float kr[16];
        float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sq = sk;
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            kr[i] = bf16_to_f32(sK[t][rg + 8 * i]);
            const float qi = bf16_to_f32(sQ[t][rg + 8 * i]);
            sk.x = fmaf(hr[i].x, kr[i], sk.x);
            sk.y = fmaf(hr[i].y, kr[i], sk.y);
            sk.z = fmaf(hr[i].z, kr[i], sk.z);
            sk.w = fmaf(hr[i].w, kr[i], sk.w);
            sq.x = fmaf(hr[i].x, qi, sq.x);
            sq.y = fmaf(hr[i].y, qi, sq.y);
            sq.z = fmaf(hr[i].z, qi, sq.z);
            sq.w = fmaf(hr[i].w, qi, sq.w);
            kq = fmaf(kr[i], qi, kq);
        }
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {   // sum over the eight row groups
            sk.x += __shfl_xor(sk.x, off);
            sk.y += __shfl_xor(sk.y, off);
            sk.z += __shfl_xor(sk.z, off);
            sk.w += __shfl_xor(sk.w, off);
            sq.x += __shfl_xor(sq.x, off);
            sq.y += __shfl_xor(sq.y, off);
            sq.z += __shfl_xor(sq.z, off);
            sq.w += __shfl_xor(sq.w, off);
            kq += __shfl_xor(kq, off);
        }
        const float4 u = make_float4(beta * (bf16_lo(vr.x) - alpha * sk.x), beta * (bf16_hi(vr.x) - alpha * sk.y),
                                     beta * (bf16_lo(vr.y) - alpha * sk.z), beta * (bf16_hi(vr.y) - alpha * sk.w));
        if (rg == 0)
            *reinterpret_cast<float4 *>(a.out + gi * D + c) =
                make_float4(fmaf(alpha, sq.x, u.x * kq), fmaf(alpha, sq.y, u.y * kq), fmaf(alpha, sq.z, u.z * kq),
                            fmaf(alpha, sq.w, u.w * kq));
        float *dst = a.node_state + gi * state_elems;
        // a leaf's state is written and the parent's stays in hr; any other
        // node's state replaces it
        const bool descend = !((leaf >> t) & 1ull);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float4 s = make_float4(fmaf(alpha, hr[i].x, kr[i] * u.x), fmaf(alpha, hr[i].y, kr[i] * u.y),
                                         fmaf(alpha, hr[i].z, kr[i] * u.z), fmaf(alpha, hr[i].w, kr[i] * u.w));
            *reinterpret_cast<float4 *>(dst + (rg + 8 * i) * D + c) = s;
            if (descend) hr[i] = s;
        }
        if (descend) held = t;
    }
}

// A plain copy of the accepted node's state, four workgroups per (request,
// head), each copying 16 KiB (more, smaller workgroups keep more of the
// stream in flight per CU than one 64 KiB workgroup).
constexpr int CQS = 4;

__global__ __launch_bounds__(NT) void commit_storeall_kernel(Args a) {
    __shared__ int s_bad;
    const int n_sub = a.B * a.Hv * CQS;
    const int sub = xcd_unit(blockIdx.x, n_sub);
    if (sub >= n_sub) return;
    const int unit = sub / CQS, q = sub - unit * CQS;
    const int b = unit / a.Hv;
    const int h = unit - b * a.Hv;
    const int tid = threadIdx.x;

    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if (st == GDN_TREE_S_OK) {
        if (tid == 0) s_bad = 0;
        __syncthreads();
        for (int t = tid; t < N; t += NT) {
            const int p = a.parent[lo + t];
            if (p < -1 || p >= t) s_bad = 1;
        }
        __syncthreads();
        if (s_bad) st = GDN_TREE_S_BAD_PARENT;
    }
    const int slot = resolve_slot(a, b);
    if (st == GDN_TREE_S_OK && slot < 0) st = GDN_TREE_S_BAD_SLOT;
    const int acc = a.accept_node[b];
    if (st == GDN_TREE_S_OK && (acc < -1 || acc >= N)) st = GDN_TREE_S_BAD_ACCEPT;
    if (h == 0 && q == 0 && tid == 0 && a.status) a.status[b] = st;
    if (slot < 0) return;
    const size_t state_elems = (size_t)D * D;
    const float *src = (st == GDN_TREE_S_OK && acc >= 0)
                           ? a.node_state_in + ((size_t)(lo + acc) * a.Hv + h) * state_elems
                           : a.S0 + ((size_t)slot * a.Hv + h) * state_elems;
    float *dst = a.S_out + ((size_t)slot * a.Hv + h) * state_elems;
    if (src == dst) return;
    const float4 *s4 = reinterpret_cast<const float4 *>(src) + q * (D * D / 4 / CQS);
    float4 *d4 = reinterpret_cast<float4 *>(dst) + q * (D * D / 4 / CQS);
#pragma unroll
    for (int i = 0; i < D * D / 4 / CQS / NT; ++i) d4[i * NT + tid] = s4[i * NT + tid];
}

}  // namespace

hipError_t launch_verify_storeall(const Args &a, hipStream_t stream) {
    const dim3 grid(xcd_grid(a.B * a.Hv)), block(NT);
    if (a.max_nodes <= 16)
        verify_storeall_kernel<16><<<grid, block, 0, stream>>>(a);
    else if (a.max_nodes <= 32)
        verify_storeall_kernel<32><<<grid, block, 0, stream>>>(a);
    else
        verify_storeall_kernel<64><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_commit_storeall(const Args &a, hipStream_t stream) {
    commit_storeall_kernel<<<dim3(xcd_grid(a.B * a.Hv * CQS)), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
