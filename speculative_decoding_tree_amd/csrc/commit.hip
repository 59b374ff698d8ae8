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
// accepted chain is the only state that gets published, and the committed
// draft is chosen on the device.  The greedy variants take that choice from
// token ids (TreeWY, "Results": greedy drafting and verification): from the
// committed root, enter the first child (index order) whose draft token equals
// the target's prediction at the current position, until none matches.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

// Greedy walk in one wave, lane t = node t (parents already validated).
// Returns the inclusive ancestor set of the accepted node (0 when none).
__device__ __forceinline__ uint64_t greedy_walk(const Args &a, int b, int lo, int N, int lane, int p,
                                                int &accept) {
    const bool live = lane < N;
    const int dtok = live ? a.draft_token[lo + lane] : 0;
    const int ttok = live ? a.target_token[lo + lane] : 0;
    int cur = -1, want = a.root_token[b];
    uint64_t pm = 0;
    for (int step = 0; step < N; ++step) {
        const uint64_t mk = __ballot(live && p == cur && dtok == want);
        if (!mk) break;
        cur = __builtin_ctzll(mk);
        pm |= 1ull << cur;
        want = __shfl(ttok, cur);
    }
    accept = cur;
    return pm;
}



constexpr int NT = 256;
constexpr int KCHUNK = 16;   // path rows staged per pass
// Workgroups per (request, head): each takes D / CQS consecutive state rows
// (16 KiB), since the rank-L update is separable by row (row i of H' needs row
// i of H0 and element i of each path k).  More, smaller workgroups keep more
// of the stream in flight per CU than one 64 KiB workgroup per unit (mixed
// batch-256: 279-280 -> 269.5-270 us, bit-identical; two per unit 270.5-271).
constexpr int CQS = 4;

// Where the accepted path comes from: the caller (a root-first path), the
// greedy walk over token ids, or the accepted node (its root-first ancestors).
enum PathSource { PATH_GIVEN = 0, PATH_GREEDY = 1, PATH_FROM_NODE = 2 };

// The workgroup's share of H0 (rows rbase .. rbase + QR - 1 of the unit's
// state) is requested first (it depends only on the slot); wave 0 then
// validates parents and the path with ballots (or derives the path: every
// share's workgroup does, one publishes it), and turns the path gates into
// decay coefficients with a suffix scan over shuffles, while those loads are
// in flight.
template <int SRC, int QS>
__global__ __launch_bounds__(NT) void commit_kernel(Args a) {
    constexpr int QR = D / QS;         // state rows of this workgroup's share
    constexpr int RI = QR / 8;         // rows per thread
    __shared__ float s_k[KCHUNK][QR];  // D_aj * k_j (this share's elements) of the current chunk
    __shared__ float s_coef[MAXN];
    __shared__ int s_path[MAXN];
    __shared__ int s_st, s_L;
    __shared__ float s_gam;

    const int n_sub = a.B * a.Hv * QS;
    const int sub = xcd_unit(blockIdx.x, n_sub);
    if (sub >= n_sub) return;
    const int unit = sub / QS, q = sub - unit * QS;
    const int rbase = q * QR;
    const int b = unit / a.Hv;
    const int h = unit - b * a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;

    const int slot = resolve_slot(a, b);
    const size_t base = ((size_t)(slot < 0 ? 0 : slot) * a.Hv + h) * D * D;
    const float4 *src = reinterpret_cast<const float4 *>(a.S0 + base);
    float4 *dst = reinterpret_cast<float4 *>(a.S_out + base);
    const int c4 = tid & 31, r0 = rbase + (tid >> 5);   // rows r0 + 8 i, columns 4 c4 .. 4 c4 + 3
    float4 acc[RI];
    if (slot >= 0) {
#pragma unroll
        for (int i = 0; i < RI; ++i) acc[i] = ld_stream4(src + (r0 + 8 * i) * 32 + c4);
    }

    if (tid < 64) {
        int lo, N;
        int st = check_offsets(a, b, lo, N);
        int L = 0;
        if (st == GDN_TREE_S_OK) {
            const bool live = lane < N;
            const int p = live ? a.parent[lo + lane] : -1;
            if (__ballot(live && (p < -1 || p >= lane))) st = GDN_TREE_S_BAD_PARENT;
        }
        if (st == GDN_TREE_S_OK && slot < 0) st = GDN_TREE_S_BAD_SLOT;
        bool have_path = false;
        int pj = 0;
        if (SRC != PATH_GIVEN) {
            int accept = -1;
            uint64_t pm = 0;
            if (SRC == PATH_FROM_NODE && st == GDN_TREE_S_OK) {
                accept = a.accept_node[b];
                if (accept < -1 || accept >= N) st = GDN_TREE_S_BAD_ACCEPT;
            }
            if (st == GDN_TREE_S_OK) {
                const int p = lane < N ? a.parent[lo + lane] : -1;
                pm = SRC == PATH_GREEDY ? greedy_walk(a, b, lo, N, lane, p, accept) : ancestors_of(lane, N, p, accept);
                L = __popcll(pm);
                pj = path_entry(pm, lane);
                have_path = true;
            }
            if (h == 0 && q == 0) {   // one head publishes the decision
                if (SRC == PATH_GREEDY && a.accept_out && lane == 0) a.accept_out[b] = accept;
                if (a.path_out) {
                    int32_t *row = a.path_out + (size_t)b * a.max_nodes;
                    if (lane < L) row[lane] = pj;
                    for (int i = L + lane; i < a.max_nodes; i += 64) row[i] = 0;
                }
                if (a.path_len_out && lane == 0) a.path_len_out[b] = L;
            }
        } else if (st == GDN_TREE_S_OK) {
            L = a.path_len[b];
            if (L < 0 || L > a.max_nodes || L > N) {
                st = GDN_TREE_S_BAD_PATH;
            } else {
                // lane j holds path entry j; it must be the child of entry j-1 (S0 for j = 0)
                const bool on = lane < L;
                pj = on ? a.path[(size_t)b * a.max_nodes + lane] : 0;
                const bool inr = on && pj >= 0 && pj < N;
                const int par = inr ? a.parent[lo + pj] : -2;
                const int prev = __shfl(pj, lane > 0 ? lane - 1 : 0);
                if (__ballot(on && (!inr || par != (lane == 0 ? -1 : prev)))) st = GDN_TREE_S_BAD_PATH;
                else have_path = true;
            }
        }
        if (have_path) {
            const bool on = lane < L;
            float coef, gam;
            path_decay(lane, L, on ? a.g[(size_t)(lo + pj) * a.Hv + h] : 0.f, coef, gam);
            if (on) {
                s_path[lane] = pj;
                s_coef[lane] = coef;   // D_aj: gates of the entries after j
            }
            if (lane == 0) s_gam = gam;
        }
        if (lane == 0) {
            s_st = st;
            s_L = L;
            if (h == 0 && q == 0 && a.status) a.status[b] = st;
        }
    }
    __syncthreads();
    const int st = s_st, L = s_L;
    if (slot < 0) return;   // nowhere to write

    if (st != GDN_TREE_S_OK || L == 0) {   // S_out = S0, bit-exact
        if (a.S_out != a.S0) {
#pragma unroll
            for (int i = 0; i < RI; ++i) st_stream4(dst + (r0 + 8 * i) * 32 + c4, acc[i]);
        }
        return;
    }

    const float gam = s_gam;
#pragma unroll
    for (int i = 0; i < RI; ++i) acc[i] = make_float4(gam * acc[i].x, gam * acc[i].y, gam * acc[i].z, gam * acc[i].w);
    int lo, N;
    check_offsets(a, b, lo, N);
    for (int j0 = 0; j0 < L; j0 += KCHUNK) {
        const int nj = min(KCHUNK, L - j0);
        if (j0 > 0) __syncthreads();
        for (int idx = tid; idx < nj * QR; idx += NT) {
            const int jj = idx / QR, c = idx - jj * QR;
            const int t = s_path[j0 + jj];
            s_k[jj][c] = s_coef[j0 + jj] * bf16_to_f32(a.k[((size_t)(lo + t) * a.Hk + hk) * D + rbase + c]);
        }
        __syncthreads();
        for (int jj = 0; jj < nj; ++jj) {
            const int t = s_path[j0 + jj];
            const float4 u = reinterpret_cast<const float4 *>(a.U + ((size_t)(lo + t) * a.Hv + h) * D)[c4];
#pragma unroll
            for (int i = 0; i < RI; ++i) {
                const float kc = s_k[jj][r0 - rbase + 8 * i];
                acc[i].x = fmaf(kc, u.x, acc[i].x);
                acc[i].y = fmaf(kc, u.y, acc[i].y);
                acc[i].z = fmaf(kc, u.z, acc[i].z);
                acc[i].w = fmaf(kc, u.w, acc[i].w);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RI; ++i) st_stream4(dst + (r0 + 8 * i) * 32 + c4, acc[i]);
}

// One wave per request, lane t = node t: parents are validated with a ballot,
// the accepted node's ancestor set comes from pointer doubling over shuffles,
// and each lane on the path writes its own entry (position = its depth - 1).
template <bool GREEDY>
__global__ __launch_bounds__(256) void accepted_path_kernel(Args a) {
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (b >= a.B) return;
    int lo, N;
    int st = check_offsets(a, b, lo, N);
    int acc = GREEDY ? -1 : a.accept_node[b];
    int32_t *row = a.path_out + (size_t)b * a.max_nodes;
    uint64_t path_mask = 0;
    if (st == GDN_TREE_S_OK) {
        const bool live = lane < N;
        const int p = live ? a.parent[lo + lane] : -1;
        if (__ballot(live && (p < -1 || p >= lane))) st = GDN_TREE_S_BAD_PARENT;
        else if (GREEDY) path_mask = greedy_walk(a, b, lo, N, lane, p, acc);
        else if (acc < -1 || acc >= N) st = GDN_TREE_S_BAD_ACCEPT;
        else if (acc >= 0) {
            int jp = p;
            uint64_t m = live ? (1ull << lane) : 0ull;
            while (__ballot(jp >= 0)) {
                const int src = jp >= 0 ? jp : lane;
                const uint64_t m_up = __shfl(m, src);
                const int jp_up = __shfl(jp, src);
                if (jp >= 0) {
                    m |= m_up;
                    jp = jp_up;
                }
            }
            path_mask = __shfl(m, acc);   // inclusive ancestors of the accepted node
        }
    }
    const int L = __popcll(path_mask);
    // the path in index order is root first; lane t on it sits at the number of path nodes below t
    if ((path_mask >> lane) & 1ull) row[__popcll(path_mask & ((1ull << lane) - 1ull))] = lane;
    for (int i = L + lane; i < a.max_nodes; i += 64) row[i] = 0;
    if (lane == 0) {
        a.path_len_out[b] = L;
        if (a.status) a.status[b] = st;
        if (GREEDY && a.accept_out) a.accept_out[b] = st == GDN_TREE_S_OK ? acc : -1;
    }
}

// gdn_tree_commit_replay: the next committed state by replaying the accepted
// path with the sequential gated delta rule from S0 (ReplaySSM, which TreeWY's
// "Prior work" names as solving the same system but materialising the state at
// another time; Tree-Scan's branch-local scan/replay).  No pseudo-values are
// read: each step computes u = beta (v - alpha S k) from the running state.
// Lane (c4, r0) keeps rows r0 + 8 i, columns 4 c4 .. +3 of the state in
// registers; S k is reduced over the 8 row groups through LDS, twice-buffered
// so one barrier per step suffices.
__global__ __launch_bounds__(NT) void replay_kernel(Args a) {
    __shared__ float s_kv[KCHUNK][2][D];      // k and v rows of the current chunk of the path
    __shared__ float4 s_part[2][8][32];       // per row-group partial sums of S k
    __shared__ int s_path[MAXN];
    __shared__ float s_alpha[MAXN], s_beta[MAXN];
    __shared__ int s_st, s_L;

    const int n_units = a.B * a.Hv;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int b = unit / a.Hv;
    const int h = unit - b * a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;

    const int slot = resolve_slot(a, b);
    const size_t base = ((size_t)(slot < 0 ? 0 : slot) * a.Hv + h) * D * D;
    const float4 *src = reinterpret_cast<const float4 *>(a.S0 + base);
    float4 *dst = reinterpret_cast<float4 *>(a.S_out + base);
    const int c4 = tid & 31, r0 = tid >> 5;   // rows r0 + 8 i, columns 4 c4 .. 4 c4 + 3
    float4 st4[16];
    if (slot >= 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) st4[i] = ld_stream4(src + (r0 + 8 * i) * 32 + c4);
    }
    int lo, N;
    if (tid < 64) {
        int st = check_offsets(a, b, lo, N);
        int L = 0;
        if (st == GDN_TREE_S_OK) {
            const bool live = lane < N;
            const int p = live ? a.parent[lo + lane] : -1;
            if (__ballot(live && (p < -1 || p >= lane))) st = GDN_TREE_S_BAD_PARENT;
        }
        if (st == GDN_TREE_S_OK && slot < 0) st = GDN_TREE_S_BAD_SLOT;
        if (st == GDN_TREE_S_OK) {
            L = a.path_len[b];
            if (L < 0 || L > a.max_nodes || L > N) {
                st = GDN_TREE_S_BAD_PATH;
            } else {
                const bool on = lane < L;
                const int pj = on ? a.path[(size_t)b * a.max_nodes + lane] : 0;
                const bool inr = on && pj >= 0 && pj < N;
                const int par = inr ? a.parent[lo + pj] : -2;
                const int prev = __shfl(pj, lane > 0 ? lane - 1 : 0);
                if (__ballot(on && (!inr || par != (lane == 0 ? -1 : prev)))) {
                    st = GDN_TREE_S_BAD_PATH;
                } else if (on) {
                    const size_t gi = (size_t)(lo + pj) * a.Hv + h;
                    s_path[lane] = pj;
                    s_alpha[lane] = expf(a.g[gi]);
                    s_beta[lane] = a.beta[gi];
                }
            }
        }
        if (lane == 0) {
            s_st = st;
            s_L = L;
            if (h == 0 && a.status) a.status[b] = st;
        }
    }
    __syncthreads();
    const int st = s_st, L = s_L;
    if (slot < 0) return;
    if (st != GDN_TREE_S_OK || L == 0) {   // S_out = S0, bit-exact
        if (a.S_out != a.S0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) st_stream4(dst + (r0 + 8 * i) * 32 + c4, st4[i]);
        }
        return;
    }
    check_offsets(a, b, lo, N);
    for (int j0 = 0; j0 < L; j0 += KCHUNK) {
        const int nj = min(KCHUNK, L - j0);
        if (j0 > 0) __syncthreads();
        for (int idx = tid; idx < nj * D; idx += NT) {
            const int jj = idx >> 7, c = idx & (D - 1);
            const int t = s_path[j0 + jj];
            s_kv[jj][0][c] = bf16_to_f32(a.k[((size_t)(lo + t) * a.Hk + hk) * D + c]);
            s_kv[jj][1][c] = bf16_to_f32(a.v[((size_t)(lo + t) * a.Hv + h) * D + c]);
        }
        __syncthreads();
        for (int jj = 0; jj < nj; ++jj) {
            const int buf = (j0 + jj) & 1;
            // partial S k over this lane's 16 rows, for its 4 columns
            float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float kr = s_kv[jj][0][r0 + 8 * i];
                part.x = fmaf(st4[i].x, kr, part.x);
                part.y = fmaf(st4[i].y, kr, part.y);
                part.z = fmaf(st4[i].z, kr, part.z);
                part.w = fmaf(st4[i].w, kr, part.w);
            }
            s_part[buf][r0][c4] = part;
            __syncthreads();
            float4 sk = s_part[buf][0][c4];
#pragma unroll
            for (int g8 = 1; g8 < 8; ++g8) {
                const float4 x = s_part[buf][g8][c4];
                sk.x += x.x;
                sk.y += x.y;
                sk.z += x.z;
                sk.w += x.w;
            }
            const float al = s_alpha[j0 + jj], be = s_beta[j0 + jj];
            const float4 vv = *reinterpret_cast<const float4 *>(&s_kv[jj][1][4 * c4]);
            const float4 u = make_float4(be * (vv.x - al * sk.x), be * (vv.y - al * sk.y),
                                         be * (vv.z - al * sk.z), be * (vv.w - al * sk.w));
#pragma unroll
            for (int i = 0; i < 16; ++i) {   // S <- alpha S + u k^T  (storage: H[i][c] = alpha H + k_i u_c)
                const float kr = s_kv[jj][0][r0 + 8 * i];
                st4[i].x = fmaf(al, st4[i].x, kr * u.x);
                st4[i].y = fmaf(al, st4[i].y, kr * u.y);
                st4[i].z = fmaf(al, st4[i].z, kr * u.z);
                st4[i].w = fmaf(al, st4[i].w, kr * u.w);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) st_stream4(dst + (r0 + 8 * i) * 32 + c4, st4[i]);
}

}  // namespace

hipError_t launch_commit_node(const Args &a, hipStream_t stream) {
    commit_kernel<PATH_FROM_NODE, CQS><<<dim3(xcd_grid(a.B * a.Hv * CQS)), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_commit(const Args &a, hipStream_t stream) {
    commit_kernel<PATH_GIVEN, CQS><<<dim3(xcd_grid(a.B * a.Hv * CQS)), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_accept_commit(const Args &a, hipStream_t stream) {
    commit_kernel<PATH_GREEDY, CQS><<<dim3(xcd_grid(a.B * a.Hv * CQS)), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_commit_replay(const Args &a, hipStream_t stream) {
    replay_kernel<<<dim3(xcd_grid(a.B * a.Hv)), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_accepted_path(const Args &a, hipStream_t stream) {
    accepted_path_kernel<false><<<dim3((a.B + 3) / 4), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_accept_greedy(const Args &a, hipStream_t stream) {
    accepted_path_kernel<true><<<dim3((a.B + 3) / 4), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
