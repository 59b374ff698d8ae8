// gdn_tree_commit and gdn_tree_accepted_path.
//
// TreeWY (arXiv 2608.20961), "Method" and "Novelty": after acceptance, only
// the accepted path's pseudo-values are composed into the next committed
// state; one full state is restored, for the accepted path only.  With the
// root-first path p_1..p_L ending at a, and D_aj = exp(sum of g over the path
// nodes after j), in storage orientation H = S^T:
//
//   H' = gamma_a H0 + sum_j D_aj k_j u_j^T
//
// a rank-L update that streams H0 in and H' out exactly once (64 KiB each per
// (request, v-head)).  GDN Tree-Scan (arXiv 2609.23900), abstract: the
// accepted chain is the only state that gets published.
#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int NT = 256;
constexpr int KCHUNK = 16;   // path rows staged per pass

__global__ __launch_bounds__(NT) void commit_kernel(Args a) {
    __shared__ float s_k[KCHUNK][D];   // D_aj * k_j rows of the current chunk
    __shared__ float s_coef[MAXN];
    __shared__ int s_path[MAXN];
    __shared__ int s_bad;
    __shared__ float s_gam;

    const int n_units = a.B * a.Hv;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int b = unit / a.Hv;
    const int h = unit - b * a.Hv;
    const int hk = h / (a.Hv / a.Hk);
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
    int L = 0;
    if (st == GDN_TREE_S_OK) {
        L = a.path_len[b];
        if (L < 0 || L > a.max_nodes || L > N) {
            st = GDN_TREE_S_BAD_PATH;
        } else {
            __syncthreads();
            if (tid == 0) {
                int prev = -1;
                for (int j = 0; j < L; ++j) {
                    const int p = a.path[(size_t)b * a.max_nodes + j];
                    if (p < 0 || p >= N || a.parent[lo + p] != prev) {
                        s_bad = 1;
                        break;
                    }
                    s_path[j] = p;
                    prev = p;
                }
                if (!s_bad) {   // suffix sums of g along the path
                    float s = 0.f;
                    for (int j = L - 1; j >= 0; --j) {
                        s_coef[j] = expf(s);
                        s += a.g[(size_t)(lo + s_path[j]) * a.Hv + h];
                    }
                    s_gam = expf(s);
                }
            }
            __syncthreads();
            if (s_bad) st = GDN_TREE_S_BAD_PATH;
        }
    }
    if (h == 0 && tid == 0 && a.status) a.status[b] = st;
    if (slot < 0) return;   // nowhere to write

    const size_t base = ((size_t)slot * a.Hv + h) * D * D;
    const float4 *src = reinterpret_cast<const float4 *>(a.S0 + base);
    float4 *dst = reinterpret_cast<float4 *>(a.S_out + base);
    const int c4 = tid & 31, r0 = tid >> 5;   // rows r0 + 8 i, columns 4 c4 .. 4 c4 + 3

    if (st != GDN_TREE_S_OK || L == 0) {   // S_out = S0, bit-exact
        if (a.S_out != a.S0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) dst[(r0 + 8 * i) * 32 + c4] = src[(r0 + 8 * i) * 32 + c4];
        }
        return;
    }

    float4 acc[16];
    const float gam = s_gam;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float4 x = src[(r0 + 8 * i) * 32 + c4];
        acc[i] = make_float4(gam * x.x, gam * x.y, gam * x.z, gam * x.w);
    }
    for (int j0 = 0; j0 < L; j0 += KCHUNK) {
        const int nj = min(KCHUNK, L - j0);
        __syncthreads();
        for (int idx = tid; idx < nj * D; idx += NT) {
            const int jj = idx >> 7, c = idx & (D - 1);
            const int t = s_path[j0 + jj];
            s_k[jj][c] = s_coef[j0 + jj] * bf16_to_f32(a.k[((size_t)(lo + t) * a.Hk + hk) * D + c]);
        }
        __syncthreads();
        for (int jj = 0; jj < nj; ++jj) {
            const int t = s_path[j0 + jj];
            const float4 u = reinterpret_cast<const float4 *>(a.U + ((size_t)(lo + t) * a.Hv + h) * D)[c4];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float kc = s_k[jj][r0 + 8 * i];
                acc[i].x = fmaf(kc, u.x, acc[i].x);
                acc[i].y = fmaf(kc, u.y, acc[i].y);
                acc[i].z = fmaf(kc, u.z, acc[i].z);
                acc[i].w = fmaf(kc, u.w, acc[i].w);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[(r0 + 8 * i) * 32 + c4] = acc[i];
}

// One lane per request: validate, then write the root-first path.
__global__ __launch_bounds__(64) void accepted_path_kernel(Args a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.B) return;
    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if (st == GDN_TREE_S_OK) {
        for (int t = 0; t < N; ++t) {
            const int p = a.parent[lo + t];
            if (p < -1 || p >= t) {
                st = GDN_TREE_S_BAD_PARENT;
                break;
            }
        }
    }
    const int acc = a.accept_node[b];
    if (st == GDN_TREE_S_OK && (acc < -1 || acc >= N)) st = GDN_TREE_S_BAD_ACCEPT;
    int32_t *row = a.path_out + (size_t)b * a.max_nodes;
    int L = 0;
    if (st == GDN_TREE_S_OK && acc >= 0) {
        for (int j = acc; j >= 0; j = a.parent[lo + j]) ++L;
        int pos = L;
        for (int j = acc; j >= 0; j = a.parent[lo + j]) row[--pos] = j;
    }
    for (int i = L; i < a.max_nodes; ++i) row[i] = 0;
    a.path_len_out[b] = L;
    if (a.status) a.status[b] = st;
}

}  // namespace

hipError_t launch_commit(const Args &a, hipStream_t stream) {
    const int n_units = a.B * a.Hv;
    commit_kernel<<<dim3(xcd_grid(n_units)), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_accepted_path(const Args &a, hipStream_t stream) {
    accepted_path_kernel<<<dim3((a.B + 63) / 64), dim3(64), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
