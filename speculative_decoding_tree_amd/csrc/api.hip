// Host side of the C ABI declared in include/gdn_tree.h: argument checks
// (nothing is enqueued when one fails), then one launch per entry point on
// the caller's stream.  The library allocates nothing and never
// synchronises.  Its only host state is a per-device cache of two launch
// facts of the attention kernel (compute units, resident workgroups per CU),
// kept in atomics and written with the same value by any thread that fills
// them.
#include <algorithm>
#include <limits.h>
#include <math.h>

#include "common.h"
#include "launch.h"

using gdn::Args;

namespace {

// Dims shared by every entry point.  need_T: whether T > 0 is meaningful.
int check_dims(const gdn_tree_dims *d) {
    if (!d) return GDN_TREE_E_NULL;
    if (d->B < 0 || d->T < 0) return GDN_TREE_E_DIMS;
    if (d->B == 0) return GDN_TREE_OK;
    if (d->Hv < 1 || d->Hk < 1 || d->Hv % d->Hk != 0 || d->n_slots < 1) return GDN_TREE_E_DIMS;
    if (d->d_k != GDN_TREE_HEAD_DIM || d->d_v != GDN_TREE_HEAD_DIM) return GDN_TREE_E_HEAD_DIM;
    if (d->max_nodes < 1 || d->max_nodes > GDN_TREE_MAX_NODES) return GDN_TREE_E_MAX_NODES;
    // one workgroup per (request, v-head), the grid rounded up to whole
    // head-group chunks per XCD (int arithmetic); indices are computed in 64-bit
    const long long units = (long long)d->B * d->Hv;
    if (units > (long long)INT_MAX / 2) return GDN_TREE_E_SIZE;
    const long long state = (long long)GDN_TREE_HEAD_DIM * GDN_TREE_HEAD_DIM * 4;
    if ((long long)d->n_slots * d->Hv > (1ll << 62) / state) return GDN_TREE_E_SIZE;
    if ((long long)d->T * d->Hv > (1ll << 62) / state) return GDN_TREE_E_SIZE;
    return GDN_TREE_OK;
}

Args base_args(const gdn_tree_dims *d) {
    Args a = {};
    a.B = d->B;
    a.Hv = d->Hv;
    a.Hk = d->Hk;
    a.T = d->T;
    a.max_nodes = d->max_nodes;
    a.n_slots = d->n_slots;
    return a;
}

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

template <typename... Ps>
bool any_misaligned(Ps... ps) {
    return (misaligned((const void *)ps) || ...);
}

// Query rows per attention workgroup.  128 (two 16-row tiles per wave, two
// workgroups per CU, blocks staged by direct loads into two LDS buffers) when
// a request can have more than 64 query rows per kv head and the scheduled
// launch takes the batch: a 64-node tree's rows then need two workgroups
// instead of four, each K and V fragment read from LDS serves 32 rows, and
// the context is read twice instead of four times; units of at most 64 rows
// still run one tile per wave.  On the batch-256 trees with 1k-4k contexts:
// 684-693 against 708-715 us for 64-row units on one GPU, and ~3.1 instead of
// 3.70 GB fetched.  Otherwise 64 (one tile per wave, three workgroups per CU;
// the waves of a one- or two-tile unit split the keys instead).  Depends only
// on the dims, so the workspace size does too.
int attn_rows_wg(const gdn_tree_attn_dims *d, int n_split) {
    const long long G = d->Hq / d->Hkv;
    const long long rows = (long long)d->max_nodes * G;
    if (rows <= 64) return 64;
    const long long n_rg = (rows + 127) / 128;
    const bool sched = (long long)d->B * n_split <= gdn::ATTN_SCHED_ITEMS && n_rg < 256 && d->Hkv * n_rg < 4096;
    return sched ? 128 : 64;
}

// split = 0: the context part size, chosen from the dims alone.  One pass
// when the batch's one-pass units (64-row count) already number
// ATTN_AUTO_UNITS; otherwise as many parts as bring the units to that count,
// at most ATTN_AUTO_PARTS (the merge reads every part of a row) and at least
// 64 keys each, rounded up to a multiple of 64 keys.  Measured on one GPU
// (one root-branch tree per request, 8 kv heads): one request with a 4096-key
// context takes 32 parts of 128 keys, 52.0 us (256-key parts 58.6, 64-key
// parts 73.5, one pass 507.8); with 16384 keys 32 parts of 512, 65.2 us (256:
// 81.0); four requests 16 parts of 256, 46.2 us; sixteen requests 4 parts of
// 1024, 64.1 us (512: 74.8).  Each was the fastest of the sizes tried.
constexpr long long ATTN_AUTO_UNITS = 512, ATTN_AUTO_PARTS = 32;
int attn_split(const gdn_tree_attn_dims *d) {
    if (d->split > 0) return d->split;
    const int one = d->max_ctx > 1 ? d->max_ctx : 1;
    const long long rows = (long long)d->max_nodes * (d->Hq / d->Hkv);
    const long long units1 = (long long)d->B * d->Hkv * ((rows + 63) / 64);
    if (units1 >= ATTN_AUTO_UNITS) return one;
    const long long parts = std::min({(ATTN_AUTO_UNITS + units1 - 1) / units1, ATTN_AUTO_PARTS,
                                      ((long long)d->max_ctx + 63) / 64});
    if (parts <= 1) return one;
    return (int)(((d->max_ctx + parts - 1) / parts + 63) / 64 * 64);
}

// Attention dims; also derives the launch shape (the context part size too).
// Returns a GDN_TREE_* code.
int check_attn_dims(const gdn_tree_attn_dims *d, int &split, int &n_split, int &n_rg) {
    split = 1;
    n_split = 1;
    n_rg = 1;
    if (!d) return GDN_TREE_E_NULL;
    if (d->B < 0 || d->T < 0 || d->C < 0) return GDN_TREE_E_DIMS;
    if (d->B == 0) return GDN_TREE_OK;
    if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv != 0) return GDN_TREE_E_DIMS;
    if (d->head_dim != GDN_TREE_HEAD_DIM) return GDN_TREE_E_HEAD_DIM;
    if (d->max_nodes < 1 || d->max_nodes > GDN_TREE_MAX_NODES) return GDN_TREE_E_MAX_NODES;
    if (d->max_ctx < 0 || d->max_ctx > (1 << 30) || d->split < 0) return GDN_TREE_E_DIMS;
    const long long G = d->Hq / d->Hkv;
    split = attn_split(d);
    n_split = d->max_ctx > split ? (int)(((long long)d->max_ctx + split - 1) / split) : 1;
    const int rows_wg = attn_rows_wg(d, n_split);
    n_rg = (int)((d->max_nodes * G + rows_wg - 1) / rows_wg);
    const long long units = (long long)d->B * d->Hkv * n_split * n_rg;
    if (units > (long long)INT_MAX - 8) return GDN_TREE_E_SIZE;
    const long long row = (long long)GDN_TREE_HEAD_DIM * 4;
    if ((long long)d->T * d->Hq > (1ll << 62) / row || (long long)d->C * d->Hkv > (1ll << 62) / row)
        return GDN_TREE_E_SIZE;
    return GDN_TREE_OK;
}

// Scheduling counters, then (split context only) one partial record per unit.
size_t attn_workspace(const gdn_tree_attn_dims *d, int n_split, int n_rg) {
    const size_t header = gdn::ATTN_WS_HEADER_BYTES;
    if (n_split <= 1) return header;
    return header + (size_t)d->B * d->Hkv * n_split * n_rg * (size_t)attn_rows_wg(d, n_split) *
                        (GDN_TREE_HEAD_DIM + 2) * sizeof(float);
}

int finish(hipError_t e) { return e == hipSuccess ? GDN_TREE_OK : GDN_TREE_E_LAUNCH; }

// Clear an error left by earlier, unrelated work so that the check after our
// launch reports our launch only.
void clear_pending() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

int gdn_tree_abi_version(void) { return GDN_TREE_ABI_VERSION; }

const char *gdn_tree_strerror(int code) {
    switch (code) {
        case GDN_TREE_OK: return "ok";
        case GDN_TREE_E_NULL: return "a required pointer is NULL";
        case GDN_TREE_E_DIMS: return "dimensions out of range (B, T, Hv, Hk, n_slots; Hv must be a multiple of Hk)";
        case GDN_TREE_E_HEAD_DIM: return "unsupported head dimension (only d_k = d_v = 128 is built)";
        case GDN_TREE_E_MAX_NODES: return "max_nodes must be in 1..64";
        case GDN_TREE_E_LAUNCH: return "kernel launch failed";
        case GDN_TREE_E_SIZE: return "buffer or grid size out of range";
        case GDN_TREE_E_ALIGN: return "state, q, k, v, out, U and node_state pointers must be 16-byte aligned";
        case GDN_TREE_E_WORKSPACE: return "attention workspace missing, misaligned or too small";
        case GDN_TREE_E_OVERLAP: return "out or U overlaps U_prev";
        case GDN_TREE_E_SCRATCH: return "the call needs more than the static scratch holds (or its address is unavailable)";
        case GDN_TREE_S_BAD_OFFSETS: return "status: node_offset out of order or beyond T";
        case GDN_TREE_S_TOO_MANY: return "status: request has more than max_nodes nodes";
        case GDN_TREE_S_BAD_PARENT: return "status: parent[t] must satisfy -1 <= parent[t] < t";
        case GDN_TREE_S_BAD_PATH: return "status: path is not a root-first chain of the request's tree";
        case GDN_TREE_S_BAD_ACCEPT: return "status: accept_node outside [-1, N_b)";
        case GDN_TREE_S_BAD_SLOT: return "status: state_slot outside [0, n_slots)";
        case GDN_TREE_S_BAD_CONTEXT: return "status: ctx_offset out of order, beyond C, or context longer than max_ctx";
        case GDN_TREE_S_BAD_MASK: return "status: an ancestry mask lacks its own node or has a later one";
        default: return "unknown gdn_tree code";
    }
}

size_t gdn_tree_state_bytes(const gdn_tree_dims *dims, int storeall) {
    if (check_dims(dims) != GDN_TREE_OK) return 0;
    const size_t rows = (size_t)dims->T * (size_t)dims->Hv;
    return storeall ? rows * (size_t)dims->d_k * (size_t)dims->d_v * 4u : rows * (size_t)dims->d_v * 4u;
}

int gdn_tree_verify(const gdn_tree_dims *dims, const float *S0, const int32_t *state_slot,
                    const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                    const float *beta, const int32_t *node_offset, const int32_t *parent, float *out,
                    float *U, uint64_t *anc_mask, int32_t *status, void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!S0 || !node_offset) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!q || !k || !v || !g || !beta || !parent || !out || !U)) return GDN_TREE_E_NULL;
    if (any_misaligned(S0, q, k, v, out, U)) return GDN_TREE_E_ALIGN;
    Args a = base_args(dims);
    a.S0 = S0;
    a.state_slot = state_slot;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.node_offset = node_offset;
    a.parent = parent;
    a.out = out;
    a.U = U;
    a.anc_mask = anc_mask;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_verify(a, (hipStream_t)stream));
}

int gdn_tree_commit(const gdn_tree_dims *dims, const float *S0, float *S_out, const int32_t *state_slot,
                    const float *U, const uint16_t *k, const float *g, const int32_t *node_offset,
                    const int32_t *parent, const int32_t *path, const int32_t *path_len, int32_t *status,
                    void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!S0 || !S_out || !node_offset || !path || !path_len) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!U || !k || !g || !parent)) return GDN_TREE_E_NULL;
    if (any_misaligned(S0, S_out, U, k)) return GDN_TREE_E_ALIGN;
    Args a = base_args(dims);
    a.S0 = S0;
    a.S_out = S_out;
    a.state_slot = state_slot;
    a.U = const_cast<float *>(U);
    a.k = k;
    a.g = g;
    a.node_offset = node_offset;
    a.parent = parent;
    a.path = path;
    a.path_len = path_len;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_commit(a, (hipStream_t)stream));
}

int gdn_tree_commit_replay(const gdn_tree_dims *dims, const float *S0, float *S_out, const int32_t *state_slot,
                           const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                           const int32_t *node_offset, const int32_t *parent, const int32_t *path,
                           const int32_t *path_len, int32_t *status, void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!S0 || !S_out || !node_offset || !path || !path_len) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!k || !v || !g || !beta || !parent)) return GDN_TREE_E_NULL;
    if (any_misaligned(S0, S_out, k, v)) return GDN_TREE_E_ALIGN;
    Args a = base_args(dims);
    a.S0 = S0;
    a.S_out = S_out;
    a.state_slot = state_slot;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.node_offset = node_offset;
    a.parent = parent;
    a.path = path;
    a.path_len = path_len;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_commit_replay(a, (hipStream_t)stream));
}

int gdn_tree_accepted_path(const gdn_tree_dims *dims, const int32_t *node_offset, const int32_t *parent,
                           const int32_t *accept_node, int32_t *path, int32_t *path_len, int32_t *status,
                           void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!node_offset || !accept_node || !path || !path_len) return GDN_TREE_E_NULL;
    if (dims->T > 0 && !parent) return GDN_TREE_E_NULL;
    Args a = base_args(dims);
    a.node_offset = node_offset;
    a.parent = parent;
    a.accept_node = accept_node;
    a.path_out = path;
    a.path_len_out = path_len;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_accepted_path(a, (hipStream_t)stream));
}

int gdn_tree_accept_greedy(const gdn_tree_dims *dims, const int32_t *node_offset, const int32_t *parent,
                           const int32_t *draft_token, const int32_t *target_token, const int32_t *root_token,
                           int32_t *accept_node, int32_t *path, int32_t *path_len, int32_t *status,
                           void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!node_offset || !root_token || !accept_node || !path || !path_len) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!parent || !draft_token || !target_token)) return GDN_TREE_E_NULL;
    Args a = base_args(dims);
    a.node_offset = node_offset;
    a.parent = parent;
    a.draft_token = draft_token;
    a.target_token = target_token;
    a.root_token = root_token;
    a.accept_out = accept_node;
    a.path_out = path;
    a.path_len_out = path_len;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_accept_greedy(a, (hipStream_t)stream));
}

int gdn_tree_accept_commit(const gdn_tree_dims *dims, const float *S0, float *S_out, const int32_t *state_slot,
                           const float *U, const uint16_t *k, const float *g, const int32_t *node_offset,
                           const int32_t *parent, const int32_t *draft_token, const int32_t *target_token,
                           const int32_t *root_token, int32_t *accept_node, int32_t *path, int32_t *path_len,
                           int32_t *status, void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!S0 || !S_out || !node_offset || !root_token) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!U || !k || !g || !parent || !draft_token || !target_token)) return GDN_TREE_E_NULL;
    if (any_misaligned(S0, S_out, U, k)) return GDN_TREE_E_ALIGN;
    Args a = base_args(dims);
    a.S0 = S0;
    a.S_out = S_out;
    a.state_slot = state_slot;
    a.U = const_cast<float *>(U);
    a.k = k;
    a.g = g;
    a.node_offset = node_offset;
    a.parent = parent;
    a.draft_token = draft_token;
    a.target_token = target_token;
    a.root_token = root_token;
    a.accept_out = accept_node;
    a.path_out = path;
    a.path_len_out = path_len;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_accept_commit(a, (hipStream_t)stream));
}

int gdn_tree_commit_node(const gdn_tree_dims *dims, const float *S0, float *S_out, const int32_t *state_slot,
                         const float *U, const uint16_t *k, const float *g, const int32_t *node_offset,
                         const int32_t *parent, const int32_t *accept_node, int32_t *path, int32_t *path_len,
                         int32_t *status, void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!S0 || !S_out || !node_offset || !accept_node) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!U || !k || !g || !parent)) return GDN_TREE_E_NULL;
    if (any_misaligned(S0, S_out, U, k)) return GDN_TREE_E_ALIGN;
    Args a = base_args(dims);
    a.S0 = S0;
    a.S_out = S_out;
    a.state_slot = state_slot;
    a.U = const_cast<float *>(U);
    a.k = k;
    a.g = g;
    a.node_offset = node_offset;
    a.parent = parent;
    a.accept_node = accept_node;
    a.path_out = path;
    a.path_len_out = path_len;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_commit_node(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Checks and argument block shared by the one-launch commit + verify entry
// points; returns a GDN_TREE_* code (GDN_TREE_OK with a.B == 0: nothing to do).
int commit_verify_args(Args &a, const gdn_tree_dims *prev_dims, const gdn_tree_dims *dims, const float *S0,
                       float *S_out, const int32_t *state_slot, const float *U_prev, const uint16_t *k_prev,
                       const float *g_prev, const int32_t *node_offset_prev, const int32_t *parent_prev,
                       int32_t *commit_status, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const float *g, const float *beta, const int32_t *node_offset, const int32_t *parent,
                       float *out, float *U, uint64_t *anc_mask, int32_t *status) {
    int rc = check_dims(prev_dims);
    if (rc != GDN_TREE_OK) return rc;
    rc = check_dims(dims);
    if (rc != GDN_TREE_OK) return rc;
    if (prev_dims->B != dims->B) return GDN_TREE_E_DIMS;
    a = base_args(dims);
    if (dims->B == 0) return GDN_TREE_OK;
    if (prev_dims->Hv != dims->Hv || prev_dims->Hk != dims->Hk || prev_dims->n_slots != dims->n_slots)
        return GDN_TREE_E_DIMS;
    if (!S0 || !S_out || !node_offset || !node_offset_prev) return GDN_TREE_E_NULL;
    if (prev_dims->T > 0 && (!U_prev || !k_prev || !g_prev || !parent_prev)) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!q || !k || !v || !g || !beta || !parent || !out || !U)) return GDN_TREE_E_NULL;
    if (any_misaligned(S0, S_out, U_prev, k_prev, q, k, v, out, U)) return GDN_TREE_E_ALIGN;
    // out and U are written while other workgroups read U_prev
    const size_t rows_prev = (size_t)prev_dims->T * dims->Hv * GDN_TREE_HEAD_DIM;
    const size_t rows = (size_t)dims->T * dims->Hv * GDN_TREE_HEAD_DIM;
    auto overlaps = [&](const float *x) {
        return x && U_prev && rows && rows_prev && x < U_prev + rows_prev && U_prev < x + rows;
    };
    if (overlaps(U) || overlaps(out)) return GDN_TREE_E_OVERLAP;
    a.S0 = S0;
    a.S_out = S_out;
    a.state_slot = state_slot;
    a.T_prev = prev_dims->T;
    a.max_nodes_prev = prev_dims->max_nodes;
    a.U_prev = U_prev;
    a.k_prev = k_prev;
    a.g_prev = g_prev;
    a.node_offset_prev = node_offset_prev;
    a.parent_prev = parent_prev;
    a.commit_status = commit_status;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.node_offset = node_offset;
    a.parent = parent;
    a.out = out;
    a.U = U;
    a.anc_mask = anc_mask;
    a.status = status;
    return GDN_TREE_OK;
}

}  // namespace

extern "C" {

int gdn_tree_commit_verify(const gdn_tree_dims *prev_dims, const gdn_tree_dims *dims, const float *S0, float *S_out,
                           const int32_t *state_slot, const float *U_prev, const uint16_t *k_prev,
                           const float *g_prev, const int32_t *node_offset_prev, const int32_t *parent_prev,
                           const int32_t *accept_node, int32_t *path, int32_t *path_len,
                           int32_t *commit_status, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const float *g, const float *beta, const int32_t *node_offset, const int32_t *parent,
                           float *out, float *U, uint64_t *anc_mask, int32_t *status, void *stream) {
    Args a;
    int rc = commit_verify_args(a, prev_dims, dims, S0, S_out, state_slot, U_prev, k_prev, g_prev, node_offset_prev,
                                parent_prev, commit_status, q, k, v, g, beta, node_offset, parent, out, U, anc_mask,
                                status);
    if (rc != GDN_TREE_OK || a.B == 0) return rc;
    if (!accept_node) return GDN_TREE_E_NULL;
    a.accept_node = accept_node;
    a.path_out = path;
    a.path_len_out = path_len;
    clear_pending();
    return finish(gdn::launch_commit_verify(a, (hipStream_t)stream));
}

int gdn_tree_accept_commit_verify(const gdn_tree_dims *prev_dims, const gdn_tree_dims *dims, const float *S0,
                                  float *S_out, const int32_t *state_slot, const float *U_prev,
                                  const uint16_t *k_prev, const float *g_prev, const int32_t *node_offset_prev,
                                  const int32_t *parent_prev, const int32_t *draft_token,
                                  const int32_t *target_token, const int32_t *root_token, int32_t *accept_node,
                                  int32_t *path, int32_t *path_len, int32_t *commit_status, const uint16_t *q,
                                  const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                                  const int32_t *node_offset, const int32_t *parent, float *out, float *U,
                                  uint64_t *anc_mask, int32_t *status, void *stream) {
    Args a;
    int rc = commit_verify_args(a, prev_dims, dims, S0, S_out, state_slot, U_prev, k_prev, g_prev, node_offset_prev,
                                parent_prev, commit_status, q, k, v, g, beta, node_offset, parent, out, U, anc_mask,
                                status);
    if (rc != GDN_TREE_OK || a.B == 0) return rc;
    if (!root_token || (prev_dims->T > 0 && (!draft_token || !target_token))) return GDN_TREE_E_NULL;
    a.draft_token = draft_token;
    a.target_token = target_token;
    a.root_token = root_token;
    a.accept_out = accept_node;
    a.path_out = path;
    a.path_len_out = path_len;
    clear_pending();
    return finish(gdn::launch_accept_commit_verify(a, (hipStream_t)stream));
}

int gdn_tree_budget_select(const gdn_tree_dims *dims, const int32_t *node_offset, const int32_t *parent,
                           const float *accept_prob, int32_t budget, float threshold, float *survival,
                           uint8_t *keep, int32_t *kept, int32_t *status, void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (dims->T >= (1 << 24)) return GDN_TREE_E_SIZE;
    if (!node_offset || !kept) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!parent || !accept_prob || !survival || !keep)) return GDN_TREE_E_NULL;
    Args a = base_args(dims);
    a.node_offset = node_offset;
    a.parent = parent;
    a.prob = accept_prob;
    a.survival = survival;
    a.keep = keep;
    a.kept = kept;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_budget_select(a, budget, threshold, (hipStream_t)stream));
}

int gdn_tree_ancestry(const gdn_tree_dims *dims, const int32_t *node_offset, const int32_t *parent,
                      uint64_t *anc_mask, int32_t *status, void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!node_offset) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!parent || !anc_mask)) return GDN_TREE_E_NULL;
    Args a = base_args(dims);
    a.node_offset = node_offset;
    a.parent = parent;
    a.anc_mask = anc_mask;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_ancestry(a, (hipStream_t)stream));
}

size_t gdn_tree_attention_workspace_bytes(const gdn_tree_attn_dims *dims) {
    int split, n_split, n_rg;
    if (check_attn_dims(dims, split, n_split, n_rg) != GDN_TREE_OK || dims->B == 0) return 0;
    return attn_workspace(dims, n_split, n_rg);
}

}  // extern "C"

namespace {

// Checks and argument block shared by the two attention entry points; `need`
// receives the workspace bytes of the launch.  Returns a GDN_TREE_* code
// (GDN_TREE_OK with a.B == 0: nothing to do).
int attention_args(gdn::AttnArgs &a, size_t &need, const gdn_tree_attn_dims *dims, const uint16_t *q,
                   const uint16_t *k_ctx, const uint16_t *v_ctx, const int32_t *ctx_offset, const uint16_t *k_node,
                   const uint16_t *v_node, const int32_t *node_offset, const uint64_t *anc_mask, float scale,
                   float *out, float *lse, int32_t *status) {
    a = {};
    need = 0;
    int split, n_split, n_rg;
    int rc = check_attn_dims(dims, split, n_split, n_rg);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!isfinite(scale) || !(scale > 0.f)) return GDN_TREE_E_DIMS;
    // per-request key/value offsets are 32-bit element counts in the kernel
    if ((long long)dims->max_ctx * dims->Hkv * GDN_TREE_HEAD_DIM >= (1ll << 31)) return GDN_TREE_E_SIZE;
    if (!node_offset || !ctx_offset) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!q || !k_node || !v_node || !anc_mask || !out)) return GDN_TREE_E_NULL;
    if (dims->C > 0 && (!k_ctx || !v_ctx)) return GDN_TREE_E_NULL;
    if (any_misaligned(q, k_ctx, v_ctx, k_node, v_node, out)) return GDN_TREE_E_ALIGN;
    need = attn_workspace(dims, n_split, n_rg);
    a.B = dims->B;
    a.Hq = dims->Hq;
    a.Hkv = dims->Hkv;
    a.G = dims->Hq / dims->Hkv;
    a.T = dims->T;
    a.C = dims->C;
    a.max_nodes = dims->max_nodes;
    a.max_ctx = dims->max_ctx;
    a.split = split;
    a.n_split = n_split;
    a.n_rg = n_rg;
    a.rows_wg = attn_rows_wg(dims, n_split);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.q = q;
    a.k_ctx = k_ctx;
    a.v_ctx = v_ctx;
    a.k_node = k_node;
    a.v_node = v_node;
    a.ctx_offset = ctx_offset;
    a.node_offset = node_offset;
    a.anc_mask = anc_mask;
    a.out = out;
    a.lse = lse;
    a.status = status;
    return GDN_TREE_OK;
}

}  // namespace

extern "C" {

int gdn_tree_attention(const gdn_tree_attn_dims *dims, const uint16_t *q, const uint16_t *k_ctx,
                       const uint16_t *v_ctx, const int32_t *ctx_offset, const uint16_t *k_node,
                       const uint16_t *v_node, const int32_t *node_offset, const uint64_t *anc_mask,
                       float scale, float *out, float *lse, void *workspace, size_t workspace_bytes,
                       int32_t *status, void *stream) {
    gdn::AttnArgs a;
    size_t need;
    int rc = attention_args(a, need, dims, q, k_ctx, v_ctx, ctx_offset, k_node, v_node, node_offset, anc_mask, scale,
                            out, lse, status);
    if (rc != GDN_TREE_OK || a.B == 0) return rc;
    if (!workspace || misaligned(workspace) || workspace_bytes < need) return GDN_TREE_E_WORKSPACE;
    a.ws = static_cast<float *>(workspace);
    clear_pending();
    return finish(gdn::launch_attention(a, (hipStream_t)stream));
}

int gdn_tree_attention_static(const gdn_tree_attn_dims *dims, const uint16_t *q, const uint16_t *k_ctx,
                              const uint16_t *v_ctx, const int32_t *ctx_offset, const uint16_t *k_node,
                              const uint16_t *v_node, const int32_t *node_offset, const uint64_t *anc_mask,
                              float scale, float *out, float *lse, int32_t *status, void *stream) {
    gdn::AttnArgs a;
    size_t need;
    int rc = attention_args(a, need, dims, q, k_ctx, v_ctx, ctx_offset, k_node, v_node, node_offset, anc_mask, scale,
                            out, lse, status);
    if (rc != GDN_TREE_OK || a.B == 0) return rc;
    if (need > GDN_TREE_STATIC_SCRATCH_BYTES) return GDN_TREE_E_SCRATCH;
    void *ws = nullptr;
    if (gdn::static_scratch(&ws) != hipSuccess || !ws) return GDN_TREE_E_SCRATCH;
    a.ws = static_cast<float *>(ws);
    clear_pending();
    return finish(gdn::launch_attention(a, (hipStream_t)stream));
}

int gdn_tree_verify_storeall(const gdn_tree_dims *dims, const float *S0, const int32_t *state_slot,
                             const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                             const float *beta, const int32_t *node_offset, const int32_t *parent,
                             float *out, float *node_state, int32_t *status, void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!S0 || !node_offset) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!q || !k || !v || !g || !beta || !parent || !out || !node_state))
        return GDN_TREE_E_NULL;
    if (any_misaligned(S0, q, k, v, out, node_state)) return GDN_TREE_E_ALIGN;
    Args a = base_args(dims);
    a.S0 = S0;
    a.state_slot = state_slot;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.node_offset = node_offset;
    a.parent = parent;
    a.out = out;
    a.node_state = node_state;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_verify_storeall(a, (hipStream_t)stream));
}

int gdn_tree_commit_storeall(const gdn_tree_dims *dims, const float *S0, float *S_out,
                             const int32_t *state_slot, const float *node_state, const int32_t *node_offset,
                             const int32_t *parent, const int32_t *accept_node, int32_t *status,
                             void *stream) {
    int rc = check_dims(dims);
    if (rc != GDN_TREE_OK || dims->B == 0) return rc;
    if (!S0 || !S_out || !node_offset || !accept_node) return GDN_TREE_E_NULL;
    if (dims->T > 0 && (!parent || !node_state)) return GDN_TREE_E_NULL;
    if (any_misaligned(S0, S_out, node_state)) return GDN_TREE_E_ALIGN;
    Args a = base_args(dims);
    a.S0 = S0;
    a.S_out = S_out;
    a.state_slot = state_slot;
    a.node_state_in = node_state;
    a.node_offset = node_offset;
    a.parent = parent;
    a.accept_node = accept_node;
    a.status = status;
    clear_pending();
    return finish(gdn::launch_commit_storeall(a, (hipStream_t)stream));
}

}  // extern "C"
