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

// Lane (c, half) owns column c and rows half*64 .. half*64+63 of every state
// it touches, so a parent state it re-reads from node_state is one it wrote.
template <int NM>
__global__ __launch_bounds__(NT) void verify_storeall_kernel(Args a) {
    __shared__ uint16_t sK[NM][D];
    __shared__ uint16_t sQ[NM][D];
    __shared__ int s_par[NM];
    __shared__ float s_red[2][D];
    __shared__ int s_bad;

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
        if (tid == 0) s_bad = 0;
        __syncthreads();
        for (int t = tid; t < N; t += NT) {
            const int p = a.parent[lo + t];
            s_par[t] = p;
            if (p < -1 || p >= t) s_bad = 1;
        }
        __syncthreads();
        if (s_bad) st = GDN_TREE_S_BAD_PARENT;
    }
    int slot = -1;
    if (st == GDN_TREE_S_OK) {
        slot = resolve_slot(a, b);
        if (slot < 0) st = GDN_TREE_S_BAD_SLOT;
    }
    if (h == 0 && tid == 0 && a.status) a.status[b] = st;
    if (st != GDN_TREE_S_OK) {
        const float qnan = __int_as_float(0x7fc00000);
        for (int idx = tid; idx < N * D; idx += NT)
            a.out[((size_t)(lo + (idx >> 7)) * a.Hv + h) * D + (idx & (D - 1))] = qnan;
        return;
    }
    for (int idx = tid; idx < N * (D / 8); idx += NT) {
        const int t = idx >> 4, c8 = idx & 15;
        const size_t row = ((size_t)(lo + t) * a.Hk + hk) * D;
        *reinterpret_cast<uint4 *>(&sK[t][c8 * 8]) = reinterpret_cast<const uint4 *>(a.k + row)[c8];
        *reinterpret_cast<uint4 *>(&sQ[t][c8 * 8]) = reinterpret_cast<const uint4 *>(a.q + row)[c8];
    }
    __syncthreads();

    const int c = tid & (D - 1), half = tid >> 7;
    const int i0 = half * 64;
    const size_t state_elems = (size_t)D * D;
    const float *H0 = a.S0 + ((size_t)slot * a.Hv + h) * state_elems;
    float hr[64];
    int held = -2;   // node whose state sits in hr (-1 = S0)
    for (int t = 0; t < N; ++t) {
        const int p = s_par[t];
        if (p != held) {
            const float *src = p < 0 ? H0 : a.node_state + ((size_t)(lo + p) * a.Hv + h) * state_elems;
#pragma unroll
            for (int m = 0; m < 64; ++m) hr[m] = src[(i0 + m) * D + c];
        }
        const size_t gi = (size_t)(lo + t) * a.Hv + h;
        const float alpha = expf(a.g[gi]);
        const float beta = a.beta[gi];
        float pk = 0.f;
#pragma unroll
        for (int m = 0; m < 64; ++m) pk = fmaf(bf16_to_f32(sK[t][i0 + m]), hr[m], pk);
        s_red[half][c] = pk;
        __syncthreads();
        const float kp = s_red[0][c] + s_red[1][c];
        const float vv = bf16_to_f32(a.v[gi * D + c]);
        const float u = beta * (vv - alpha * kp);
        __syncthreads();
        float *dst = a.node_state + gi * state_elems;
        float po = 0.f;
#pragma unroll
        for (int m = 0; m < 64; ++m) {
            const float x = fmaf(alpha, hr[m], bf16_to_f32(sK[t][i0 + m]) * u);
            hr[m] = x;
            dst[(i0 + m) * D + c] = x;
            po = fmaf(bf16_to_f32(sQ[t][i0 + m]), x, po);
        }
        s_red[half][c] = po;
        __syncthreads();
        if (half == 0) a.out[gi * D + c] = s_red[0][c] + s_red[1][c];
        __syncthreads();
        held = t;
    }
}

__global__ __launch_bounds__(NT) void commit_storeall_kernel(Args a) {
    __shared__ int s_bad;
    const int n_units = a.B * a.Hv;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
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
    if (h == 0 && tid == 0 && a.status) a.status[b] = st;
    if (slot < 0) return;
    const size_t state_elems = (size_t)D * D;
    const float *src = (st == GDN_TREE_S_OK && acc >= 0)
                           ? a.node_state_in + ((size_t)(lo + acc) * a.Hv + h) * state_elems
                           : a.S0 + ((size_t)slot * a.Hv + h) * state_elems;
    float *dst = a.S_out + ((size_t)slot * a.Hv + h) * state_elems;
    if (src == dst) return;
    const float4 *s4 = reinterpret_cast<const float4 *>(src);
    float4 *d4 = reinterpret_cast<float4 *>(dst);
#pragma unroll
    for (int i = 0; i < 16; ++i) d4[i * NT + tid] = s4[i * NT + tid];
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
    commit_storeall_kernel<<<dim3(xcd_grid(a.B * a.Hv)), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
