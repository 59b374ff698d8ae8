/*
 * gdn_tree.h -- C ABI of the tree-structured Gated DeltaNet speculative
 * verification library (libgdn_tree.so, gfx950 / MI355X).
 *
 * What the library computes
 * -------------------------
 * A Gated DeltaNet layer keeps, per value head, a fixed-size recurrent state
 * S (d_v x d_k) and advances it one token at a time with the gated delta rule
 *
 *     alpha_t = exp(g_t)
 *     u_t     = beta_t * (v_t - alpha_t * S_{t-1} k_t)      (pseudo-value)
 *     S_t     = alpha_t * S_{t-1} + u_t k_t^T,    o_t = S_t q_t
 *
 * (TreeWY, arXiv 2608.20961: "Background" and "Method"; the pseudo-value is
 * the new value minus what the decayed preceding state already predicts).
 * For tree speculative decoding, every draft node must see the state that
 * sequential decode would produce along its root-to-node path (GDN Tree-Scan,
 * arXiv 2609.23900, abstract).  gdn_tree_verify computes every node's output
 * and pseudo-value at once from the committed state S0 with an ancestor-masked
 * unit-lower-triangular solve (TreeWY, "Method" and "Novelty": tree-structured
 * WY transform, one triangular system, parent-before-child order).
 * gdn_tree_commit rebuilds only the accepted path's state from the same
 * pseudo-values (TreeWY, "Novelty": one full state is restored for the
 * accepted path; Tree-Scan: accepted-chain-only state publication).  The
 * *_storeall entry points are the snapshot-per-node scheme kept for
 * comparison (TreeWY, "Prior work": vLLM's storeall saves the committed state
 * plus one state per candidate position and selects the accepted one).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer except `dims` is a DEVICE pointer (HIP device memory of the
 *   current device) unless stated otherwise.  The caller owns all buffers;
 *   the library never allocates, frees or synchronises.  Each call enqueues
 *   kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 * - Only d_k = d_v = 128 is compiled.  Smaller heads run zero-padded to 128,
 *   which is exact (padded coordinates never interact).
 * - Layouts are dense row-major:
 *     S0, S_out   float32 [n_slots][Hv][d_k][d_v]: the state stored transposed
 *                 (H = S^T): row i holds what the state returns for key e_i.
 *     state_slot  int32 [B]: slot of request b in S0/S_out; NULL = slot b.
 *                 Entry points that write S_out need distinct slots (two
 *                 requests on one slot would write it concurrently).
 *     q, k        bfloat16 bit patterns (uint16) [T][Hk][d_k]
 *     v           bfloat16 bit patterns [T][Hv][d_v]
 *     g, beta     float32 [T][Hv]: log-decay g <= 0 (alpha = exp(g)) and beta
 *     node_offset int32 [B+1]: request b owns node rows node_offset[b] ..
 *                 node_offset[b+1]-1; node_offset[B] must equal T
 *     parent      int32 [T]: request-local parent index, -1 = attached to S0;
 *                 parent[t] < t (parent-before-child; a forest is allowed)
 *     out, U      float32 [T][Hv][d_v]: node outputs and pseudo-values
 *                 (beta folded into U)
 *     anc_mask    uint64 [T]: inclusive ancestor bitset, bit j = request-local
 *                 node j
 *     path        int32 [B][max_nodes]: root-first request-local node indices
 *     path_len    int32 [B]: 0 = nothing accepted
 *     accept_node int32 [B]: last accepted node, -1 = none
 *     node_state  float32 [T][Hv][d_k][d_v] (storeall only)
 *     status      int32 [B] (optional, may be NULL): per-request device status
 * - S0, S_out, q, k, v, out, U and node_state must be 16-byte aligned (the
 *   kernels move them in 16-byte vectors); other arrays need natural alignment.
 * - v-head h reads key head h / (Hv / Hk) (grouped-query heads).
 * - Return value: 0 = enqueued; a negative GDN_TREE_E_* code = rejected on
 *   the host and NOTHING was enqueued.  Problems only visible on the device
 *   are reported per request in status[b] (GDN_TREE_S_*); the documented
 *   fallback output is written for that request instead.
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_TREE_ABI_VERSION 3   /* 2: gdn_tree_commit_verify, gdn_tree_accept_commit_verify, GDN_TREE_E_OVERLAP;
                                    3: gdn_tree_attention_static, GDN_TREE_E_SCRATCH */
#define GDN_TREE_MAX_NODES 64   /* per request: one wave64 lane and one uint64 bit per node */
#define GDN_TREE_HEAD_DIM 128

/* host-side return codes (nothing enqueued) */
#define GDN_TREE_OK 0
#define GDN_TREE_E_NULL (-1)      /* a required pointer is NULL */
#define GDN_TREE_E_DIMS (-2)      /* B, T, Hv, Hk, n_slots out of range or Hv % Hk != 0 */
#define GDN_TREE_E_HEAD_DIM (-3)  /* d_k or d_v is not 128 */
#define GDN_TREE_E_MAX_NODES (-4) /* max_nodes < 1 or > 64 */
#define GDN_TREE_E_LAUNCH (-5)    /* the HIP runtime refused the launch */
#define GDN_TREE_E_SIZE (-6)      /* a buffer would exceed 2^62 bytes */
#define GDN_TREE_E_ALIGN (-7)     /* a state / q / k / v / out / U / node_state pointer is not 16-byte aligned */
#define GDN_TREE_E_WORKSPACE (-8) /* attention workspace missing, misaligned or smaller than required */
#define GDN_TREE_E_OVERLAP (-9)   /* gdn_tree_commit_verify: out or U overlaps U_prev */
#define GDN_TREE_E_SCRATCH (-10)  /* gdn_tree_attention_static: the call needs more than the static scratch holds,
                                     or the scratch's device address could not be obtained */

/* Bytes of the per-device static scratch of gdn_tree_attention_static. */
#define GDN_TREE_STATIC_SCRATCH_BYTES (64u << 20)

/* device-side per-request status codes (status[b]) */
#define GDN_TREE_S_OK 0
#define GDN_TREE_S_BAD_OFFSETS 1  /* node_offset[b] < 0, decreasing, or node_offset[b+1] > T */
#define GDN_TREE_S_TOO_MANY 2     /* request has more than max_nodes nodes */
#define GDN_TREE_S_BAD_PARENT 3   /* some parent[t] >= t or < -1 */
#define GDN_TREE_S_BAD_PATH 4     /* path is not a root-first chain of the tree, or path_len out of range */
#define GDN_TREE_S_BAD_ACCEPT 5   /* accept_node outside [-1, N_b) */
#define GDN_TREE_S_BAD_SLOT 6     /* state_slot[b] outside [0, n_slots) */
#define GDN_TREE_S_BAD_CONTEXT 7  /* ctx_offset[b] < 0, decreasing, beyond C, or context longer than max_ctx */
#define GDN_TREE_S_BAD_MASK 8     /* some anc_mask[t] lacks bit t or has a bit above t */

typedef struct gdn_tree_dims {
    int32_t B;         /* requests in the batch (>= 0) */
    int32_t Hv;        /* value heads (>= 1) */
    int32_t Hk;        /* key heads (>= 1, divides Hv) */
    int32_t d_k;       /* key head dim, must be 128 */
    int32_t d_v;       /* value head dim, must be 128 */
    int32_t T;         /* total draft nodes = node_offset[B] (>= 0) */
    int32_t max_nodes; /* per-request node cap and row stride of path[] (1..64) */
    int32_t n_slots;   /* slots in S0 / S_out (>= 1 when B > 0) */
} gdn_tree_dims;

/*
 * gdn_tree_verify -- outputs and pseudo-values of every draft node.
 *
 * For each request b and v-head h, with anc*(t) the inclusive ancestors of t,
 * G_t the sum of g over anc*(t), gamma_t = exp(G_t) and D_tj = exp(G_t - G_j):
 *   U solves  u_t + beta_t * sum_{j in anc(t)} D_tj (k_t.k_j) u_j
 *                 = beta_t * (v_t - gamma_t * S0 k_t)
 *   out_t = gamma_t * S0 q_t + sum_{j in anc*(t)} D_tj (q_t.k_j) u_j
 * which equals sequential decode along each root-to-node path (TreeWY,
 * "Method"; Tree-Scan, abstract).  No per-node state is materialised.
 *
 * Reads S0, state_slot, q, k, v, g, beta, node_offset, parent; writes out, U,
 * anc_mask (if non-NULL) and status (if non-NULL).  state_slot, anc_mask and
 * status may be NULL; q, k, v, g, beta, parent, out, U may be NULL when T == 0.
 * Device errors: a request with bad offsets is skipped (status 1); a request
 * with too many nodes or a bad parent array gets NaN rows in out and U and
 * zero ancestry masks (status 2 / 3); a bad slot gives NaN rows (status 6).
 */
int gdn_tree_verify(const gdn_tree_dims *dims, const float *S0, const int32_t *state_slot,
                    const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                    const float *beta, const int32_t *node_offset, const int32_t *parent,
                    float *out, float *U, uint64_t *anc_mask, int32_t *status, void *stream);

/*
 * gdn_tree_commit -- the next committed state from the accepted path only.
 *
 * For the root-first path p_1..p_L ending at node a (L = path_len[b]):
 *   S_out = gamma_a * S0 + sum_{j in path} D_aj u_j k_j^T     (stored transposed)
 * i.e. the sequential state at node a (TreeWY, "Method": only the accepted
 * path's pseudo-values are composed into the next committed state).  L = 0
 * copies S0 bit-exactly.  S_out may alias S0 (in-place commit).  U must be the
 * pseudo-values gdn_tree_verify produced for the same inputs.
 * Device errors: an invalid path (status 4) or an invalid request (1..3) makes
 * S_out[slot] a copy of S0[slot]; a bad slot (6) writes nothing.
 */
int gdn_tree_commit(const gdn_tree_dims *dims, const float *S0, float *S_out,
                    const int32_t *state_slot, const float *U, const uint16_t *k, const float *g,
                    const int32_t *node_offset, const int32_t *parent, const int32_t *path,
                    const int32_t *path_len, int32_t *status, void *stream);

/*
 * gdn_tree_commit_replay -- the next committed state by replaying the accepted
 * path with the sequential gated delta rule from S0, without pseudo-values:
 * for each path node in order, u = beta (v - alpha S k), S <- alpha S + u k^T
 * (ReplaySSM, named in TreeWY's "Prior work"; GDN Tree-Scan, abstract:
 * branch-local scan/replay).  Reads k, v, g, beta of the path nodes instead of
 * U.  Same path format, statuses and fallbacks as gdn_tree_commit; L = 0
 * copies S0 bit-exactly; S_out may alias S0.
 */
int gdn_tree_commit_replay(const gdn_tree_dims *dims, const float *S0, float *S_out,
                           const int32_t *state_slot, const uint16_t *k, const uint16_t *v, const float *g,
                           const float *beta, const int32_t *node_offset, const int32_t *parent,
                           const int32_t *path, const int32_t *path_len, int32_t *status, void *stream);

/*
 * gdn_tree_accepted_path -- root-first path from each request's accepted node.
 *
 * path[b][0..L) = the nodes from the S0-attached root down to accept_node[b]
 * (Tree-Scan: accepted chain), path_len[b] = L; the rest of the row is zeroed.
 * accept_node[b] = -1 gives L = 0.  Device errors (status 1..3, 5) give L = 0.
 */
int gdn_tree_accepted_path(const gdn_tree_dims *dims, const int32_t *node_offset,
                           const int32_t *parent, const int32_t *accept_node, int32_t *path,
                           int32_t *path_len, int32_t *status, void *stream);

/*
 * gdn_tree_accept_greedy -- greedy acceptance on the device.
 *
 * Per request, starting at the committed root whose target prediction is
 * root_token[b]: among the current position's children in index order, enter
 * the first whose draft_token equals the target's prediction at the current
 * position (target_token[t] after node t), until none matches (TreeWY,
 * "Results": greedy drafting and verification; GDN Tree-Scan, abstract:
 * device-side choice of the committed draft).  Writes accept_node[b] (-1 when
 * the first level already fails), the root-first path (zero-filled row) and
 * path_len.  draft_token, target_token int32 [T] and root_token int32 [B] are
 * arbitrary token ids.  Device errors (status 1..3) give accept_node = -1,
 * path_len = 0.
 */
int gdn_tree_accept_greedy(const gdn_tree_dims *dims, const int32_t *node_offset, const int32_t *parent,
                           const int32_t *draft_token, const int32_t *target_token,
                           const int32_t *root_token, int32_t *accept_node, int32_t *path,
                           int32_t *path_len, int32_t *status, void *stream);

/*
 * gdn_tree_commit_node -- gdn_tree_accepted_path fused with gdn_tree_commit,
 * in one launch: each (request, v-head) workgroup derives the root-first path
 * of accept_node[b] (int32 [B], request-local, -1 = nothing accepted) in one
 * wave while its H0 is being read, then composes that path's pseudo-values
 * into S_out exactly as gdn_tree_commit does (TreeWY, "Method": only the
 * accepted path is composed into the next state).  path [B][max_nodes] and
 * path_len [B] are optional outputs (NULL = not written), identical to what
 * gdn_tree_accepted_path writes.  Device errors: bad offsets (1), too many
 * nodes (2), bad parent (3), bad slot (6), accept_node outside [-1, N_b) (5);
 * the request's S_out is then a copy of S0 (nothing is written where the slot
 * is bad), and its path is empty.
 */
int gdn_tree_commit_node(const gdn_tree_dims *dims, const float *S0, float *S_out,
                         const int32_t *state_slot, const float *U, const uint16_t *k, const float *g,
                         const int32_t *node_offset, const int32_t *parent, const int32_t *accept_node,
                         int32_t *path, int32_t *path_len, int32_t *status, void *stream);

/*
 * gdn_tree_commit_verify -- the commit of the previous tree's accepted node
 * and the verify of the next tree, in one launch.
 *
 * In a decoding loop the state committed for one draft tree is the state the
 * next tree is verified from (TreeWY, "Method": only the accepted path is
 * composed into the next committed state, and verification starts from the
 * committed state).  Each (request, v-head) workgroup reads S0 once, composes
 * the previous tree's accepted path into it as gdn_tree_commit_node does,
 * writes the result to S_out, and verifies the next tree from the registers
 * that hold it, so the committed state is not read back.  Results equal
 * gdn_tree_commit_node(prev_dims, S0 -> S_out, U_prev, k_prev, g_prev,
 * node_offset_prev, parent_prev, accept_node) followed by
 * gdn_tree_verify(dims, S_out, ...) bit for bit.
 *
 * prev_dims describes the previous tree (its T and max_nodes); B, Hv, Hk and
 * n_slots must equal those of dims (GDN_TREE_E_DIMS otherwise).  U_prev,
 * k_prev, g_prev, node_offset_prev and parent_prev are that tree's
 * pseudo-values (from its verify), keys, gates, offsets and parents, in the
 * layouts above; accept_node int32 [B] is its accepted node (-1 = none).
 * The other arguments are those of gdn_tree_verify for the next tree.
 * S_out may alias S0 (in place: nothing is written for a request with an
 * empty path); out and U must not overlap U_prev (GDN_TREE_E_OVERLAP).
 * commit_status [B] (optional) receives the commit's device status as
 * gdn_tree_commit_node reports it, status [B] the verify's.  path
 * [B][prev max_nodes] and path_len [B] (optional, NULL = not written) receive
 * the previous tree's accepted root-first path as gdn_tree_accepted_path
 * writes it (for moving the accepted nodes' attention KV rows, for example).  A request whose
 * commit fails (bad offsets, parent or accept_node) is verified from S0,
 * which is also what S_out then holds; a bad slot writes nothing and gives
 * NaN outputs, as the two calls would.
 */
int gdn_tree_commit_verify(const gdn_tree_dims *prev_dims, const gdn_tree_dims *dims, const float *S0,
                           float *S_out, const int32_t *state_slot, const float *U_prev,
                           const uint16_t *k_prev, const float *g_prev, const int32_t *node_offset_prev,
                           const int32_t *parent_prev, const int32_t *accept_node, int32_t *path,
                           int32_t *path_len, int32_t *commit_status, const uint16_t *q, const uint16_t *k,
                           const uint16_t *v, const float *g, const float *beta, const int32_t *node_offset,
                           const int32_t *parent, float *out, float *U, uint64_t *anc_mask, int32_t *status,
                           void *stream);

/*
 * gdn_tree_accept_commit_verify -- gdn_tree_commit_verify with the previous
 * tree's accepted node chosen on the device by the greedy walk of
 * gdn_tree_accept_greedy (TreeWY, "Results": greedy drafting and
 * verification; GDN Tree-Scan, abstract: device-side choice of the committed
 * draft), in the same launch: the acceptance, the commit and the next tree's
 * verify take one launch per layer.  draft_token and target_token (int32
 * [T_prev]) and root_token (int32 [B]) are the previous tree's token ids as
 * gdn_tree_accept_greedy takes them; accept_node (int32 [B], optional output)
 * receives the node the walk accepted (-1 when none, or on a commit error).
 * Results equal gdn_tree_accept_commit followed by gdn_tree_verify bit for
 * bit; everything else is as in gdn_tree_commit_verify.
 */
int gdn_tree_accept_commit_verify(const gdn_tree_dims *prev_dims, const gdn_tree_dims *dims, const float *S0,
                                  float *S_out, const int32_t *state_slot, const float *U_prev,
                                  const uint16_t *k_prev, const float *g_prev, const int32_t *node_offset_prev,
                                  const int32_t *parent_prev, const int32_t *draft_token,
                                  const int32_t *target_token, const int32_t *root_token, int32_t *accept_node,
                                  int32_t *path, int32_t *path_len, int32_t *commit_status, const uint16_t *q,
                                  const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                                  const int32_t *node_offset, const int32_t *parent, float *out, float *U,
                                  uint64_t *anc_mask, int32_t *status, void *stream);

/*
 * gdn_tree_accept_commit -- greedy acceptance fused with the commit, in one
 * launch: each (request, v-head) workgroup repeats the greedy walk of
 * gdn_tree_accept_greedy (one wave, no host round trip) and composes that
 * path's pseudo-values into S_out exactly as gdn_tree_commit does.
 * accept_node, path and path_len are optional outputs (NULL = not written).
 * Device errors as in gdn_tree_commit (bad path cannot occur).
 */
int gdn_tree_accept_commit(const gdn_tree_dims *dims, const float *S0, float *S_out,
                           const int32_t *state_slot, const float *U, const uint16_t *k, const float *g,
                           const int32_t *node_offset, const int32_t *parent, const int32_t *draft_token,
                           const int32_t *target_token, const int32_t *root_token, int32_t *accept_node,
                           int32_t *path, int32_t *path_len, int32_t *status, void *stream);

/*
 * gdn_tree_budget_select -- load-adaptive choice of the draft nodes to verify.
 *
 * survival[t] = product of accept_prob over t's root-to-node path, formed in
 * float32 root first (s = s_parent * p) (DSpark adaptive verification: per-token
 * acceptance -> per-position survival; TreeSpark: a branch's value).  Nodes of
 * all valid requests are ordered by survival descending, then depth, then
 * global index; the first `budget` of them with survival >= threshold get
 * keep[t] = 1 (DSpark: a global budget to the positions with the highest
 * survival across requests; TreeSpark: growth stops below a threshold).  Every
 * ancestor of a kept node is kept.  kept[b] counts request b's kept nodes.
 * accept_prob float32 [T] must lie in [0, 1]; survival float32 [T]; keep
 * uint8 [T]; kept int32 [B].  Invalid requests (status 1..3) get NaN survival
 * and no kept node.  Requires T < 2^24.  Three small launches; no workspace.
 */
int gdn_tree_budget_select(const gdn_tree_dims *dims, const int32_t *node_offset, const int32_t *parent,
                           const float *accept_prob, int32_t budget, float threshold, float *survival,
                           uint8_t *keep, int32_t *kept, int32_t *status, void *stream);

/*
 * gdn_tree_ancestry -- inclusive ancestor bitsets of every draft node.
 *
 * anc_mask[t] (uint64 [T]) has bit j set for every request-local node j on
 * t's root-to-node path, t included (TreeWY, "Method": parent-before-child
 * order, a node couples only to its ancestors).  One set per forward pass
 * serves every attention layer (gdn_tree_attention) and equals the masks
 * gdn_tree_verify writes.  Uses B, T and max_nodes of dims (the other fields
 * are validated as for every entry point).  Device errors: bad offsets (1)
 * write nothing; too many nodes or a bad parent (2, 3) write zero masks.
 */
int gdn_tree_ancestry(const gdn_tree_dims *dims, const int32_t *node_offset, const int32_t *parent,
                      uint64_t *anc_mask, int32_t *status, void *stream);

/* Dimensions of the tree-bias attention entry points. */
typedef struct gdn_tree_attn_dims {
    int32_t B;         /* requests (>= 0) */
    int32_t Hq;        /* query heads (>= 1, a multiple of Hkv) */
    int32_t Hkv;       /* key/value heads (>= 1); query head h reads kv head h / (Hq / Hkv) */
    int32_t head_dim;  /* must be 128 */
    int32_t T;         /* total draft nodes = node_offset[B] (>= 0) */
    int32_t C;         /* total committed-context rows = ctx_offset[B] (>= 0) */
    int32_t max_nodes; /* per-request node cap (1..64) */
    int32_t max_ctx;   /* per-request context cap (0 .. 2^30) */
    int32_t split;     /* context keys per workgroup; split >= max_ctx = one pass, no merge;
                          0 = chosen by the library from these dims: one pass when B * Hkv * row groups
                          of 64 reaches 512, else min(ceil(512 / those units), 32, ceil(max_ctx / 64))
                          parts, each ceil(max_ctx / parts) rounded up to a multiple of 64 keys (one
                          pass if that is a single part); one request with a 4096-token context and
                          8 kv heads: 32 parts of 128 keys */
} gdn_tree_attn_dims;

/*
 * gdn_tree_attention -- ancestry-masked (tree-bias) decode attention for the
 * attention layers of a hybrid model over a draft forest.
 *
 * Row (t, h) of draft node t attends to every key of its request's committed
 * context and to the draft nodes in anc_mask[t] (its inclusive ancestors):
 * exactly what sequential decode of t's root-to-node path sees (GDN
 * Tree-Scan, abstract: attention layers need only an ancestry mask, applied
 * as tree-bias attention).  With s_j = scale * (q_t,h . key_j):
 *   out[t][h] = sum_j softmax(s)_j value_j,    lse[t][h] = log sum_j exp(s_j)
 * Layouts (bfloat16 bit patterns unless stated):
 *   q              [T][Hq][128]
 *   k_ctx, v_ctx   [C][Hkv][128]; request b's context is rows ctx_offset[b] ..
 *                  ctx_offset[b+1]-1 (int32 [B+1], ctx_offset[B] = C)
 *   k_node, v_node [T][Hkv][128]: the draft nodes' own keys and values
 *   anc_mask       uint64 [T] as written by gdn_tree_ancestry
 *   out            float32 [T][Hq][128];  lse float32 [T][Hq] (may be NULL)
 * When split < max_ctx the context is cut into ceil(max_ctx / split) parts
 * handled by separate workgroups and merged by a second launch.  Every call
 * with B > 0 needs a caller-owned device workspace of
 * gdn_tree_attention_workspace_bytes(dims) bytes (16-byte aligned; contents
 * need no initialisation): 256 bytes of work-distribution counters, which the
 * call zeroes on the stream itself, followed, for a split context, by the
 * parts' partial results.  Calls that share a workspace must not overlap.
 * q, k_ctx, v_ctx, k_node, v_node and out must be 16-byte aligned.  scale must be finite and positive.  max_ctx * Hkv * 128
 * must stay below 2^31 (GDN_TREE_E_SIZE otherwise).
 * Device errors: bad node offsets (1) write nothing for the request; too
 * many nodes (2), a bad context range (7) or a malformed mask (8) give NaN
 * rows in out and lse.
 */
int gdn_tree_attention(const gdn_tree_attn_dims *dims, const uint16_t *q, const uint16_t *k_ctx,
                       const uint16_t *v_ctx, const int32_t *ctx_offset, const uint16_t *k_node,
                       const uint16_t *v_node, const int32_t *node_offset, const uint64_t *anc_mask,
                       float scale, float *out, float *lse, void *workspace, size_t workspace_bytes,
                       int32_t *status, void *stream);

/* Workspace bytes gdn_tree_attention needs for dims: 256 for one pass; for a
 * split context 256 + B * Hkv * parts * row groups * rows * 130 * 4, where a
 * row group holds rows = 128 query rows when max_nodes * Hq / Hkv > 64 and
 * B * parts <= 1024, else 64; 0 when B = 0 or dims are invalid.  Host only. */
size_t gdn_tree_attention_workspace_bytes(const gdn_tree_attn_dims *dims);

/*
 * gdn_tree_attention_static -- gdn_tree_attention without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments (minus workspace and workspace_bytes), results and error
 * behaviour as gdn_tree_attention, bit for bit.  The work-distribution
 * counters and the partial results of a split context live in a static device
 * array of GDN_TREE_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on
 * every GPU it runs on until the process ends; the call allocates nothing.
 * Its first call on a device looks up that device's copy of the array.  A
 * call whose workspace need (gdn_tree_attention_workspace_bytes) exceeds the
 * array returns GDN_TREE_E_SCRATCH and enqueues nothing: one pass always
 * fits (256 bytes); a split context fits while B * Hkv * parts * row groups
 * partial records fit: 2016 records of 64 rows (33,280 bytes each), or 1008
 * of 128 rows (66,560 bytes), the size taken when a request and kv head have
 * more than 64 query rows (max_nodes * Hq / Hkv) and B * parts <= 1024.
 * Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (concurrent streams, or
 * graphs replayed concurrently) race and must be serialised by the caller.
 * The counters are cleared on the stream by each call; partial records are
 * written before they are read, so nothing left by an earlier call is used.
 */
int gdn_tree_attention_static(const gdn_tree_attn_dims *dims, const uint16_t *q, const uint16_t *k_ctx,
                              const uint16_t *v_ctx, const int32_t *ctx_offset, const uint16_t *k_node,
                              const uint16_t *v_node, const int32_t *node_offset, const uint64_t *anc_mask,
                              float scale, float *out, float *lse, int32_t *status, void *stream);

/*
 * gdn_tree_verify_storeall -- the snapshot-per-node comparison scheme.
 *
 * Walks each request's nodes in order with the sequential rule and writes
 * every node's full state (TreeWY, "Prior work": storeall keeps one state per
 * candidate position; a tree needs one per node):
 *   node_state[t] = (alpha_t S_parent + u_t k_t^T)^T,   out_t = S_t q_t.
 * Same inputs and error behaviour as gdn_tree_verify (NaN rows in out; the
 * node states of a failed request are left unwritten).
 */
int gdn_tree_verify_storeall(const gdn_tree_dims *dims, const float *S0, const int32_t *state_slot,
                             const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *g, const float *beta, const int32_t *node_offset,
                             const int32_t *parent, float *out, float *node_state,
                             int32_t *status, void *stream);

/*
 * gdn_tree_commit_storeall -- copy the accepted node's snapshot into S_out
 * (S0 when accept_node[b] == -1).  S_out may alias S0.  Device errors (1..3,
 * 5) copy S0; a bad slot (6) writes nothing.
 */
int gdn_tree_commit_storeall(const gdn_tree_dims *dims, const float *S0, float *S_out,
                             const int32_t *state_slot, const float *node_state,
                             const int32_t *node_offset, const int32_t *parent,
                             const int32_t *accept_node, int32_t *status, void *stream);

/*
 * gdn_tree_state_bytes -- speculative recurrent-state bytes one layer holds
 * beyond S0, for the memory comparison of the two schemes.  storeall != 0
 * gives T*Hv*d_k*d_v*4: one fp32 state per node and head (TreeWY, "Prior
 * work": storeall keeps the committed state plus one state per candidate
 * position, so a depth-3 chain needs four).  storeall == 0 gives the fp32
 * pseudo-value matrix U, T*Hv*d_v*4 (TreeWY, "Novelty": one small
 * pseudo-value matrix replaces the per-node states, and one full state is
 * rebuilt for the accepted path only).  Host only; 0 on invalid dims.
 */
size_t gdn_tree_state_bytes(const gdn_tree_dims *dims, int storeall);

/* Static description of a return or status code (host only, never NULL). */
const char *gdn_tree_strerror(int code);

/* GDN_TREE_ABI_VERSION of the built library (host only). */
int gdn_tree_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_H */
