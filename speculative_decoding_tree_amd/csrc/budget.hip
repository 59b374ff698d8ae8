// gdn_tree_budget_select: the load-adaptive choice of the nodes to verify.
//
// DSpark adaptive verification (news page on the vLLM feature): estimate each
// draft token's acceptance probability, derive each position's survival
// probability, and give a global budget B of positions to those with the
// highest survival across requests, on the GPU.  TreeSpark: a tree grows
// best-first along the most promising branch and stops once the best
// remaining value falls below a threshold.  Here:
//   s_t = s_parent(t) * p_t   (float32, root first; s_root = p_root)
//   order: s descending, then depth, then global node index (unique keys)
//   keep = first `budget` nodes of that order with s >= threshold.
// Kernel 1 (one wave per request) validates the tree and forms survival and
// depth level by level; kernel 2 (one workgroup) radix-selects the
// budget-th smallest 64-bit key (~bits(s), depth, index) in eight 8-bit
// passes and marks the kept nodes.
#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

__global__ __launch_bounds__(256) void survival_kernel(Args a) {
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (b >= a.B) return;
    int lo, N;
    int st = check_offsets(a, b, lo, N);
    const bool live = st == GDN_TREE_S_OK && lane < N;
    const int p = live ? a.parent[lo + lane] : -1;
    if (st == GDN_TREE_S_OK && __ballot(live && (p < -1 || p >= lane))) st = GDN_TREE_S_BAD_PARENT;
    if (st == GDN_TREE_S_OK) {
        const float pt = live ? a.prob[lo + lane] : 0.f;
        float s = pt;
        int dep = live && p < 0 ? 1 : 0;                // 0 = not reached yet
        // level by level: a node whose parent is done multiplies the parent's survival
        while (__ballot(live && dep == 0)) {
            const float sp = __shfl(s, p < 0 ? lane : p);
            const int dp = __shfl(dep, p < 0 ? lane : p);
            if (live && dep == 0 && dp > 0) {
                s = sp * pt;
                dep = dp + 1;
            }
        }
        if (live) {
            a.survival[lo + lane] = s;
            a.keep[lo + lane] = (uint8_t)dep;   // depth for now; select_kernel overwrites it with the flag
        }
    } else if (st != GDN_TREE_S_BAD_OFFSETS) {
        for (int t = lane; t < N; t += 64) {
            a.survival[lo + t] = __int_as_float(0x7fc00000);
            a.keep[lo + t] = 0;   // invalid request: never selected
        }
    }
    if (lane == 0 && a.status) a.status[b] = st;
}

// Sort key of node t: ascending key = survival descending, then depth, then index.
// Survival is in [0, 1] (non-negative floats order like their bit patterns).
__device__ __forceinline__ uint64_t node_key(float s, int dep, int t) {
    if (dep == 0) return ~0ull;   // invalid request: after everything
    const uint32_t sb = __float_as_uint(s);
    return ((uint64_t)(~sb) << 32) | ((uint64_t)dep << 24) | (uint64_t)t;
}

constexpr int SEL_T = 1024;
constexpr int SEL_KPT = 8;   // keys a thread keeps in registers across the passes (T <= 8192)

__global__ __launch_bounds__(SEL_T) void select_kernel(Args a, int budget, float threshold) {
    __shared__ uint32_t hist[256];
    __shared__ uint64_t s_prefix;
    __shared__ int s_rank;
    const int tid = threadIdx.x;
    const float *surv = a.survival;
    const uint8_t *dep = a.keep;
    uint8_t *keep = a.keep;
    const int T = a.T;
    // budget-th smallest key (1-based); none when budget <= 0, all when budget >= T
    uint64_t kth = 0;
    const bool all = budget >= T;
    const bool cached = T <= SEL_T * SEL_KPT;
    uint64_t kc[SEL_KPT];
#pragma unroll
    for (int j = 0; j < SEL_KPT; ++j) {
        const int t = tid + j * SEL_T;
        kc[j] = (cached && t < T) ? node_key(surv[t], dep[t], t) : ~0ull;
    }
    if (budget > 0 && !all) {
        if (tid == 0) {
            s_prefix = 0;
            s_rank = budget;
        }
        __syncthreads();
        for (int pass = 7; pass >= 0; --pass) {
            const int shift = 8 * pass;
            const uint64_t hi_mask = pass == 7 ? 0ull : (~0ull << (shift + 8));
            for (int i = tid; i < 256; i += SEL_T) hist[i] = 0;
            __syncthreads();
            const uint64_t prefix = s_prefix;
            if (cached) {
#pragma unroll
                for (int j = 0; j < SEL_KPT; ++j)
                    if (tid + j * SEL_T < T && (kc[j] & hi_mask) == prefix)
                        atomicAdd(&hist[(kc[j] >> shift) & 0xff], 1u);
            } else {
                for (int t = tid; t < T; t += SEL_T) {
                    const uint64_t key = node_key(surv[t], dep[t], t);
                    if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xff], 1u);
                }
            }
            __syncthreads();
            if (tid < 64) {
                // wave 0 finds the digit holding the rank: lane l sums bins 4l .. 4l+3,
                // an inclusive scan over lanes gives each lane's cumulative count, and
                // the first lane whose cumulative count reaches the rank owns the digit
                const int r = s_rank;
                const uint32_t h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2],
                               h3 = hist[4 * tid + 3];
                int incl = (int)(h0 + h1 + h2 + h3);
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int up = __shfl_up(incl, off);
                    if (tid >= off) incl += up;
                }
                const int excl = incl - (int)(h0 + h1 + h2 + h3);
                const unsigned long long hit = __ballot(incl >= r);
                const int owner = __ffsll((long long)hit) - 1;   // r <= total, so some lane hits
                if (tid == owner) {
                    int rr = r - excl, d = 4 * tid;
                    if ((int)h0 < rr) {
                        rr -= h0;
                        ++d;
                        if ((int)h1 < rr) {
                            rr -= h1;
                            ++d;
                            if ((int)h2 < rr) {
                                rr -= h2;
                                ++d;
                            }
                        }
                    }
                    s_rank = rr;
                    s_prefix = prefix | ((uint64_t)d << shift);
                }
            }
            __syncthreads();
        }
        kth = s_prefix;
    }
    for (int t = tid; t < T; t += SEL_T) {
        const int d = dep[t];
        const uint64_t key = node_key(surv[t], d, t);
        const bool sel = d > 0 && budget > 0 && (all || key <= kth) && surv[t] >= threshold;
        keep[t] = sel ? 1 : 0;   // same element this lane just read its depth from
    }
}

__global__ __launch_bounds__(256) void count_kernel(Args a) {
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (b >= a.B) return;
    int lo, N;
    const int st = check_offsets(a, b, lo, N);
    int c = 0;
    if (st == GDN_TREE_S_OK) {
        c = __popcll(__ballot(lane < N && a.keep[lo + lane]));
    }
    if (lane == 0) a.kept[b] = c;
}

}  // namespace

hipError_t launch_budget_select(const Args &a, int budget, float threshold, hipStream_t stream) {
    const dim3 g4((a.B + 3) / 4);
    survival_kernel<<<g4, dim3(256), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    select_kernel<<<dim3(1), dim3(SEL_T), 0, stream>>>(a, budget, threshold);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    count_kernel<<<g4, dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
