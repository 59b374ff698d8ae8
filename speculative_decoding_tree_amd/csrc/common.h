// Device helpers shared by the gfx950 kernels of libgdn_tree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn_tree.h"

namespace gdn {

constexpr int D = GDN_TREE_HEAD_DIM;   // d_k = d_v = 128
constexpr int MAXN = GDN_TREE_MAX_NODES;
// Attention workspace: scheduling counters first, then the partial records of
// a split context.
constexpr int ATTN_WS_HEADER_BYTES = 256;
// The scheduled attention launch builds its unit list in LDS: at most this
// many (request, context part) items.
constexpr int ATTN_SCHED_ITEMS = 1024;

// Plain-old-data argument block shared by every launcher.
struct Args {
    int B, Hv, Hk, T, max_nodes, n_slots;
    const float *S0;
    float *S_out;
    const int32_t *state_slot;
    const uint16_t *q, *k, *v;
    const float *g, *beta;
    const int32_t *node_offset, *parent;
    float *out, *U;
    uint64_t *anc_mask;
    int32_t *status;
    const int32_t *path, *path_len, *accept_node;
    int32_t *path_out, *path_len_out;
    float *node_state;
    const float *node_state_in;
    const int32_t *draft_token, *target_token, *root_token;
    int32_t *accept_out;
    const float *prob;      // budget selection: acceptance probabilities [T]
    float *survival;        // [T]
    uint8_t *keep;          // [T]
    int32_t *kept;          // [B]
    // gdn_tree_commit_verify: the previous tree, whose accepted path is
    // committed before the current tree is verified
    int T_prev, max_nodes_prev;
    const float *U_prev, *g_prev;
    const uint16_t *k_prev;
    const int32_t *node_offset_prev, *parent_prev;
    int32_t *commit_status;
};

// Argument block of the tree-bias attention kernels.
struct AttnArgs {
    int B, Hq, Hkv, G, T, C, max_nodes, max_ctx, split, n_split, n_rg;
    int rows_wg;                            // query rows per workgroup (64 or 128)
    float scale_log2;                       // softmax scale times log2(e)
    const uint16_t *q, *k_ctx, *v_ctx, *k_node, *v_node;
    const int32_t *ctx_offset, *node_offset;
    const uint64_t *anc_mask;
    float *out, *lse, *ws;
    int32_t *status;
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Streaming accesses: each byte of a committed state is touched once per
// call, so loads and stores carry the non-temporal hint (no cache retention).
__device__ __forceinline__ float2 ld_stream2(const float *p) {
    const f32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x2_t *>(p));
    return make_float2(v.x, v.y);
}
__device__ __forceinline__ float4 ld_stream4(const float4 *p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream4(float4 *p, float4 x) {
    __builtin_nontemporal_store(f32x4_t{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4_t *>(p));
}
__device__ __forceinline__ void st_stream2(float *p, float2 x) {
    __builtin_nontemporal_store(f32x2_t{x.x, x.y}, reinterpret_cast<f32x2_t *>(p));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// low / high bf16 of a packed pair, widened exactly
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Offsets check for request b of a tree with T rows: returns a GDN_TREE_S_*
// code and the row range.
__device__ __forceinline__ int check_offsets_at(const int32_t *node_offset, int T, int max_nodes, int b, int &lo,
                                                int &n) {
    lo = node_offset[b];
    const int hi = node_offset[b + 1];
    n = hi - lo;
    if (lo < 0 || hi < lo || hi > T) return GDN_TREE_S_BAD_OFFSETS;
    if (n > max_nodes) return GDN_TREE_S_TOO_MANY;
    return GDN_TREE_S_OK;
}

__device__ __forceinline__ int check_offsets(const Args &a, int b, int &lo, int &n) {
    return check_offsets_at(a.node_offset, a.T, a.max_nodes, b, lo, n);
}

// Inclusive ancestor set of node acc (one wave, lane t = node t, p = parent of
// node t or -1 past the tree, parents validated), by pointer doubling over
// shuffles; 0 for acc = -1.
__device__ __forceinline__ uint64_t ancestors_of(int lane, int N, int p, int acc) {
    const bool live = lane < N;
    int jp = live ? p : -1;
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
    return acc >= 0 ? __shfl(m, acc) : 0ull;
}

// Node at position `lane` (root first) of the path set pm, or 0 past its end.
__device__ __forceinline__ int path_entry(uint64_t pm, int lane) {
    uint64_t m = pm;
    for (int k = 0; k < lane && m; ++k) m &= m - 1;
    return m ? __builtin_ctzll(m) : 0;
}

// Decay of a root-first path of L entries, entry j in lane j with its gate
// gj: coef = exp(sum of g over the entries after j) (D_aj for the last entry
// a) and gam = exp(sum of g over the whole path) (gamma_a), from a suffix
// scan over shuffles.  Every commit kernel forms them this way, so their
// results agree bit for bit.
__device__ __forceinline__ void path_decay(int lane, int L, float gj, float &coef, float &gam) {
    const bool on = lane < L;
    float sfx = on ? gj : 0.f;
    const float g0 = sfx;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float up = __shfl_down(sfx, off);
        if (lane + off < 64) sfx += up;
    }
    coef = expf(sfx - g0);
    gam = expf(__shfl(sfx, 0));
}

__device__ __forceinline__ int resolve_slot(const Args &a, int b) {
    const int s = a.state_slot ? a.state_slot[b] : b;
    return (s < 0 || s >= a.n_slots) ? -1 : s;
}

// Map a linear workgroup id to a (request, v-head) unit so that the Hv/Hk
// v-heads sharing one key head, and neighbouring requests, run on the same
// XCD: workgroups are dispatched round-robin over the 8 XCDs, so id w runs on
// XCD w % 8; each XCD gets one contiguous range of units.
__device__ __forceinline__ int xcd_unit(int w, int n_units) {
    const int per = (n_units + 7) >> 3;
    return (w & 7) * per + (w >> 3);
}

__host__ __device__ __forceinline__ int xcd_grid(int n_units) { return ((n_units + 7) >> 3) << 3; }

// Head-group-interleaved mapping: the r = Hv/Hk v-heads that share a key head
// form a head group; chunks of C consecutive head groups (b Hk + g) are dealt
// round-robin over the 8 XCDs (workgroup w runs on XCD w % 8).  Every XCD
// gets the same share of every request's heads (exactly when Hk is a
// multiple of 8 C), whatever the mix of tree sizes; the v-heads of a group
// run one after another on one XCD, where their q and k rows meet in L2; and
// a chunk's states are contiguous.  C = 2 when Hk is a multiple of 16, else 1
// (measured on 16 key heads: C = 2 beats 1 and 4).  Returns the unit b Hv + h,
// or -1 for a slot past the last group.
__device__ __forceinline__ int xcd_group_unit(int w, int B, int Hk, int r) {
    const int cs = (Hk & 15) == 0 ? 1 : 0;   // log2 C
    const int x = w & 7, s = w >> 3;
    const int qi = s / r, j = s - qi * r;   // this XCD's qi-th head group, v-head j of it
    const int ch = qi >> cs, wi = qi - (ch << cs);
    const int q = ((ch * 8 + x) << cs) + wi;
    return q < B * Hk ? q * r + j : -1;
}

__host__ __device__ __forceinline__ int xcd_group_grid(int B, int Hk, int r) {
    const int C = (Hk & 15) == 0 ? 2 : 1;
    return 8 * ((B * Hk + 8 * C - 1) / (8 * C)) * C * r;
}

}  // namespace gdn
