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

// Offsets check for request b: returns a GDN_TREE_S_* code and the row range.
__device__ __forceinline__ int check_offsets(const Args &a, int b, int &lo, int &n) {
    lo = a.node_offset[b];
    const int hi = a.node_offset[b + 1];
    n = hi - lo;
    if (lo < 0 || hi < lo || hi > a.T) return GDN_TREE_S_BAD_OFFSETS;
    if (n > a.max_nodes) return GDN_TREE_S_TOO_MANY;
    return GDN_TREE_S_OK;
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

}  // namespace gdn
