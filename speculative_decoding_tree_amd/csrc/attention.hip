// gdn_tree_ancestry and gdn_tree_attention: the draft tree's ancestry bitsets
// and the attention layers' tree-bias decode attention.
//
// GDN Tree-Scan (abstract): in one target pass over a draft tree, the
// attention layers need only an ancestry mask (tree-bias attention); the
// recurrent layers need the per-path state (the verify kernels).  Row (t, h)
// attends to the request's committed context and to t's inclusive ancestors
// among the draft nodes, which is what sequential decode along t's
// root-to-node path attends to.
//
// gfx950 layout.  A workgroup (4 wave64) owns 64 query rows of one
// (request, kv-head), or 128 (two 16-row tiles per wave) when a request can
// have more than 64 rows per kv head: row r = (node r / G, query head
// hk G + r % G), so the G query heads of a node sit in neighbouring rows and
// every row of the workgroup shares the same keys.  Each group of 16 rows is
// owned by one wave.  Keys go through LDS 64 at a time, K and V rows as they are in
// memory, their 16-byte chunks permuted per row (XOR) so that fragment reads
// hit distinct banks.  Per block and wave:
//   S^T = K Q^T          (v_mfma_f32_16x16x32_bf16; A = K rows from LDS,
//                         B = the wave's Q rows, loaded once into registers)
// leaves lane (n, grp) with keys 16kt + 4grp + i of query row n, so the
// online-softmax statistics of row n live in the four lanes of row n, and
// the probabilities are already laid out as the B operand of
//   O^T += V^T P^T       (A = V^T, read from the row-major V block with the
//                         transposing LDS read ds_read_b64_tr_b16; k-slot
//                         8grp + e holds key 32ks + 16(e/4) + 4grp + e%4 in both)
// with P split into bf16 hi + lo (two MFMAs, ~16 mantissa bits), so no
// register moves between lanes.  Blocks wholly inside the context skip the
// mask; a row's running max only moves when a block raises it by more than
// 2^8, so most blocks need no cross-lane reduction.  Loads of the next block
// are issued before the current block is computed (into registers with
// 64-row units, straight into a second LDS buffer with 128-row units).
//
// When a request's context is split over several workgroups, each writes an
// unnormalised partial (O, running max, sum) to the workspace and a second
// kernel merges them.
#include <math.h>

#include <atomic>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace gdn {
namespace {

// ---- ancestry ------------------------------------------------------------

// One wave per request, lane t = node t.  Pointer doubling: m is the set of
// nodes from t up to (excluding) jp; each round joins the segment above.
__global__ __launch_bounds__(256) void ancestry_kernel(Args a) {
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (b >= a.B) return;
    int lo, N;
    int st = check_offsets(a, b, lo, N);
    if (st == GDN_TREE_S_BAD_OFFSETS) {
        if (lane == 0 && a.status) a.status[b] = st;
        return;
    }
    const bool live = st == GDN_TREE_S_OK && lane < N;
    int jp = live ? a.parent[lo + lane] : -1;
    if (st == GDN_TREE_S_OK && __ballot(live && (jp < -1 || jp >= lane))) st = GDN_TREE_S_BAD_PARENT;
    uint64_t m = 0ull;
    if (st == GDN_TREE_S_OK) {
        m = live ? (1ull << lane) : 0ull;
        while (__ballot(jp >= 0)) {
            const int src = jp >= 0 ? jp : lane;
            const uint64_t m_up = __shfl(m, src);
            const int jp_up = __shfl(jp, src);
            if (jp >= 0) {
                m |= m_up;
                jp = jp_up;
            }
        }
    }
    for (int t = lane; t < N; t += 64) a.anc_mask[lo + t] = st == GDN_TREE_S_OK ? m : 0ull;
    if (lane == 0 && a.status) a.status[b] = st;
}

// ---- attention -------------------------------------------------------------

constexpr int AT = 256;              // threads per workgroup
constexpr int KB = 64;               // keys per staged block
// K and V blocks sit in LDS row-major (one 256-byte row per key) with the
// sixteen 16-byte chunks of a row permuted by an XOR with a function of the
// row, so that the fragment reads below hit distinct banks.
__device__ __forceinline__ int k_at(int row, int c) { return row * D + 8 * (c ^ (row & 15)); }
__device__ __forceinline__ int v_at(int row, int c) { return row * D + 8 * (c ^ ((row & 7) << 1)); }

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane 4a + b receives
// element b of the 8 bytes addressed by lanes a, 4 + a, 8 + a, 12 + a.  p is
// restrict (nothing else writes what it reads while the read runs): with that
// the compiler does not hold the read for direct LDS loads in flight into
// another buffer, which the callers wait for themselves.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t *__restrict__ p) {
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(p));
    return __builtin_bit_cast(u32x2, r);
}
// A workgroup owns rows_wg = 64 TPW query rows (TPW 16-row tiles per wave); a
// partial record of a split context holds rows_wg rows of O, then the
// rows' running max, then their sums.
__host__ __device__ __forceinline__ size_t part_floats(int rows_wg) { return (size_t)rows_wg * (D + 2); }
constexpr float LN2 = 0.6931471805599453f;
// The running max of a row is only moved when a block raises it by more than
// this many powers of two; until then probabilities stay below 2^RESCALE.
constexpr float RESCALE = 8.f;

// Request checks shared by both kernels: offsets, node count, context range.
__device__ __forceinline__ int attn_request(const AttnArgs &a, int b, int &lo, int &N, int &c0, int &Lc) {
    lo = a.node_offset[b];
    const int hi = a.node_offset[b + 1];
    N = hi - lo;
    c0 = 0;
    Lc = 0;
    if (lo < 0 || hi < lo || hi > a.T) return GDN_TREE_S_BAD_OFFSETS;
    if (N > a.max_nodes) return GDN_TREE_S_TOO_MANY;
    c0 = a.ctx_offset[b];
    const int c1 = a.ctx_offset[b + 1];
    Lc = c1 - c0;
    if (c0 < 0 || c1 < c0 || c1 > a.C || Lc > a.max_ctx) return GDN_TREE_S_BAD_CONTEXT;
    return GDN_TREE_S_OK;
}

// A node's mask must hold the node itself and nothing after it.  Uniform per
// workgroup (every thread calls the barrier).
__device__ __forceinline__ int check_masks(const AttnArgs &a, int st, int lo, int N) {
    if (st != GDN_TREE_S_OK || N == 0) return st;
    const int t = threadIdx.x;
    const bool bad = t < N && (a.anc_mask[lo + t] >> t) != 1ull;
    return __syncthreads_or(bad) ? GDN_TREE_S_BAD_MASK : st;
}

// NaN out / lse rows [r_begin, r_end) of (request at lo, kv-head hk), all threads.
__device__ void nan_rows(const AttnArgs &a, int lo, int hk, int r_begin, int r_end) {
    const float qnan = __int_as_float(0x7fc00000);
    const int G = a.G;
    for (int idx = threadIdx.x; idx < (r_end - r_begin) * D; idx += AT) {
        const int r = r_begin + idx / D, t = r / G, g = r - t * G;
        a.out[((size_t)(lo + t) * a.Hq + hk * G + g) * D + (idx & (D - 1))] = qnan;
    }
    if (a.lse)
        for (int i = threadIdx.x; i < r_end - r_begin; i += AT) {
            const int r = r_begin + i, t = r / G, g = r - t * G;
            a.lse[(size_t)(lo + t) * a.Hq + hk * G + g] = qnan;
        }
}

// Rows a workgroup of row group rg answers for when the request is invalid:
// its own rows, and for the last group every row beyond (a request with more
// nodes than max_nodes has rows no group was sized for).
__device__ __forceinline__ int nan_end(const AttnArgs &a, int rg, int R) {
    return rg == a.n_rg - 1 ? R : min(R, a.rows_wg * (rg + 1));
}

// The block loop of one unit.  KG waves share each 16-row tile, wave
// (tile, group) taking keys [KB g / KG, KB (g + 1) / KG) of every block; the
// groups' running (max, sum, O) are merged at the end through LDS.  KG = 1 is
// the plain layout (one tile per wave, every key); units of one or two tiles
// use KG = 4 or 2 so that no wave idles.  RROWS is the launch's unit size (64
// or 128 rows): the layout of its partial records, and with 128 the staging
// by direct loads into two LDS buffers.
template <int TPW, int KG, int RROWS>
__device__ __forceinline__ void attn_body(const AttnArgs &a, int b, int hk, int sp, int rg, int rot, uint16_t *Ks,
                                          uint16_t *Vs, uint16_t *Ks2, uint16_t *Vs2, uint32_t *vnf_all, int lo,
                                          int N, int c0, int R, int row0, int k0, int k1, int nctx, int nblk);

// One unit: query rows [ROWS rg, ROWS (rg + 1)) of (request b, kv-head hk)
// against context part sp (and, for part 0, the draft nodes).  Ks / Vs are
// the workgroup's LDS block (Ks2 / Vs2 the second one of 128-row units) and
// vnf_all its per-thread record of non-finite node values; rot only varies
// which wave takes which rows.
template <int TPW>
__device__ __forceinline__ void attn_unit(const AttnArgs &a, int b, int hk, int sp, int rg, int rot, uint16_t *Ks,
                                          uint16_t *Vs, uint16_t *Ks2, uint16_t *Vs2, uint32_t *vnf_all) {
    constexpr int ROWS = 64 * TPW;
    const int tid = threadIdx.x;

    int lo, N, c0, Lc;
    int st = attn_request(a, b, lo, N, c0, Lc);
    st = check_masks(a, st, lo, N);
    if (hk == 0 && sp == 0 && rg == 0 && tid == 0 && a.status) a.status[b] = st;
    if (st == GDN_TREE_S_BAD_OFFSETS) return;
    const int G = a.G;
    const int R = N * G;
    const int row0 = ROWS * rg;
    if (row0 >= R) return;
    if (st != GDN_TREE_S_OK) {   // NaN rows (the merge kernel writes them when the context is split)
        if (a.n_split == 1) nan_rows(a, lo, hk, row0, nan_end(a, rg, R));
        return;
    }
    const int k0 = sp * a.split;
    if (sp > 0 && k0 >= Lc) return;   // nothing of this request's context falls in this part
    const int k1 = min(Lc, k0 + a.split);
    const int nctx = k1 > k0 ? (k1 - k0 + KB - 1) / KB : 0;
    const int nblk = nctx + (sp == 0 ? 1 : 0);   // the draft nodes' own block goes with the first part
    // A unit with at most 64 rows (every unit of a 64-row launch, and in a
    // 128-row launch small requests and a request's last row group) runs one
    // tile per wave, its waves sharing a tile through key groups when it has
    // one or two; its partial record keeps the launch's row count.
    const int tiles = (min(R - row0, ROWS) + 15) >> 4;
    if (tiles == 1)
        attn_body<1, 4, ROWS>(a, b, hk, sp, rg, rot, Ks, Vs, Ks2, Vs2, vnf_all, lo, N, c0, R, row0, k0, k1, nctx, nblk);
    else if (tiles == 2)
        attn_body<1, 2, ROWS>(a, b, hk, sp, rg, rot, Ks, Vs, Ks2, Vs2, vnf_all, lo, N, c0, R, row0, k0, k1, nctx, nblk);
    else if (TPW == 1 || tiles <= 4)
        attn_body<1, 1, ROWS>(a, b, hk, sp, rg, rot, Ks, Vs, Ks2, Vs2, vnf_all, lo, N, c0, R, row0, k0, k1, nctx, nblk);
    else if constexpr (TPW > 1)
        attn_body<TPW, 1, ROWS>(a, b, hk, sp, rg, rot, Ks, Vs, Ks2, Vs2, vnf_all, lo, N, c0, R, row0, k0, k1, nctx, nblk);
}

template <int TPW, int KG, int RROWS>
__device__ __forceinline__ void attn_body(const AttnArgs &a, int b, int hk, int sp, int rg, int rot, uint16_t *Ks,
                                          uint16_t *Vs, uint16_t *Ks2, uint16_t *Vs2, uint32_t *vnf_all, int lo,
                                          int N, int c0, int R, int row0, int k0, int k1, int nctx, int nblk) {
    static_assert(RROWS >= 64 * TPW, "a partial record holds the unit's rows");
    static_assert(KG == 1 || TPW == 1, "key groups split one tile per wave");
    constexpr int NKT = 4 / KG;            // this wave's 16-key tiles per block
    constexpr int NKS = NKT >= 2 ? NKT / 2 : 1;   // its 32-key value steps
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // lane values are recomputed per unit, not held across a resident loop
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), n = lane & 15, grp = lane >> 4;
    const int G = a.G;
    // ---- this lane's query rows (MFMA B column n), one per tile ----
    // With KG = 1, row slot wr of the group goes to wave (wr + rot) % 4, so that
    // groups with a single slot do not all compute on the same wave slot.
    const int wr = KG > 1 ? w / KG : (w - rot) & 3;
    const int kg = KG > 1 ? w % KG : 0;   // key group
    const int kt_lo = kg * NKT;            // first 16-key tile of the block this wave takes
    // A wave computes its second tile even when the tile has no valid row (a
    // unit's last wave): its rows are never written, and the products stay
    // free of branches, which lets the compiler interleave them.
    int t[TPW], g[TPW];
    bool rvalid[TPW], tact[TPW];   // tact: the tile has a valid row (wave-uniform)
    uint64_t anc_row[TPW];
    u32x4 qf[TPW][4];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int rb = row0 + 16 * (TPW * wr + tt);
        const int r = rb + n;
        tact[tt] = rb < R;
        rvalid[tt] = r < R;
        t[tt] = rvalid[tt] ? r / G : 0;
        g[tt] = rvalid[tt] ? r - t[tt] * G : 0;
        anc_row[tt] = rvalid[tt] ? a.anc_mask[lo + t[tt]] : 0ull;
        if (rvalid[tt]) {
            const uint16_t *qp = a.q + ((size_t)(lo + t[tt]) * a.Hq + hk * G + g[tt]) * D + 8 * grp;
#pragma unroll
            for (int s = 0; s < 4; ++s) qf[tt][s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) qf[tt][s] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    const bool active = tact[0];
    // Two tiles per wave leave no registers to spare: there the rows' ancestry
    // masks and output indices are derived again where they are used (the
    // draft nodes' block and the end) rather than held across the blocks.
    auto row_index = [&](int tt, int &tr, int &gr) {
        if constexpr (TPW == 1) {
            tr = t[tt];
            gr = g[tt];
        } else {
            int id = threadIdx.x;
            asm volatile("" : "+v"(id));
            const int r = row0 + 16 * (TPW * wr + tt) + (id & 15);
            tr = rvalid[tt] ? r / G : 0;
            gr = rvalid[tt] ? r - tr * G : 0;
        }
    };
    auto ancestry = [&](int tt) -> uint64_t {
        if constexpr (TPW == 1) {
            return anc_row[tt];
        } else {
            int tr, gr;
            row_index(tt, tr, gr);
            return rvalid[tt] ? a.anc_mask[lo + tr] : 0ull;
        }
    };

    // ---- staging: 16 lanes per row and 16-byte chunk c = tid % 16, so each
    //      load instruction reads whole rows; thread tid moves rows 16q + tid / 16
    //      of K and of V, q = 0..3. ----
    const int cch = tid & 15, srow = tid >> 4;
    // per-request bases are workgroup-uniform; lanes add 32-bit element offsets
    // (a request's context is below 2^31 elements per array, checked on the host)
    const uint32_t kvrow = (uint32_t)a.Hkv * D;
    const uint16_t *kctx = a.k_ctx + ((size_t)c0 * a.Hkv + hk) * D;
    const uint16_t *vctx = a.v_ctx + ((size_t)c0 * a.Hkv + hk) * D;
    const uint16_t *knode = a.k_node + ((size_t)lo * a.Hkv + hk) * D;
    const uint16_t *vnode = a.v_node + ((size_t)lo * a.Hkv + hk) * D;
    // The 128-row launch (two workgroups per CU) has LDS for two blocks: it
    // stages by direct global-to-LDS loads into the other buffer while a block
    // is computed, which frees the staging registers.  One wave instruction
    // fills four rows (lane l: row 4 j + l / 16, LDS chunk l % 16, written at
    // the row's base + 16 l); the lane loads the global chunk that the swizzle
    // puts there.  The 64-row launches stage through registers.
    constexpr bool DMA = RROWS == 128;
    u32x4 kst[4], vst[4];
    // Wave w fills rows 4 j .. 4 j + 3, j = w + 4 i (i = 0..3); lane l takes row
    // r = 16 i + r0, r0 = 4 w + l % 64 / 16.  r % 16 = r0 % 16 for every i, so
    // the swizzled chunk (byte offset ck for K, cv for V) is fixed per lane.
    const int r0 = 4 * w + ((tid & 63) >> 4);
    const uint32_t ck = 16u * (uint32_t)((tid & 15) ^ (r0 & 15));
    const uint32_t cv = 16u * (uint32_t)((tid & 15) ^ ((r0 & 7) << 1));
    const uint32_t rowb = 2u * kvrow;   // bytes between consecutive rows of one kv head
    auto issue_block = [&](int blk, uint16_t *Kd, uint16_t *Vd) {
        const bool nodeb = blk >= nctx;
        const int last = nodeb ? N - 1 : k1 - 1;
        const int first = nodeb ? 0 : k0 + KB * blk;
        const char *kb = reinterpret_cast<const char *>(nodeb ? knode : kctx);
        const char *vb = reinterpret_cast<const char *>(nodeb ? vnode : vctx);
        const bool whole = first + KB - 1 <= last;   // no row past the end (workgroup-uniform)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = w + 4 * i;
            // 32-bit byte offsets from a uniform base (a request's rows stay below
            // 2^31 elements, so 2^32 bytes, per array: checked on the host)
            const uint32_t ro = whole ? (uint32_t)(first + r0) * rowb + (uint32_t)(16 * i) * rowb
                                      : (uint32_t)min(first + 16 * i + r0, last) * rowb;
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4 *>(kb + (ro + ck)),
                                             (__attribute__((address_space(3))) void *)&Kd[4 * j * D], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4 *>(vb + (ro + cv)),
                                             (__attribute__((address_space(3))) void *)&Vd[4 * j * D], 16, 0, 0);
        }
    };
    auto load_block = [&](int blk) {
        const bool nodeb = blk >= nctx;
        // key rows past the end read the last real row; their scores are masked
        const int last = nodeb ? N - 1 : k1 - 1;
        const int first = nodeb ? 0 : k0 + KB * blk;
        const uint16_t *kb = nodeb ? knode : kctx;
        const uint16_t *vb = nodeb ? vnode : vctx;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t off = (uint32_t)min(first + 16 * q + srow, last) * kvrow + 8 * cch;
            kst[q] = *reinterpret_cast<const u32x4 *>(kb + off);
            vst[q] = *reinterpret_cast<const u32x4 *>(vb + off);
        }
    };
    auto store_block = [&]() {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<u32x4 *>(&Ks[k_at(16 * q + srow, cch)]) = kst[q];
            *reinterpret_cast<u32x4 *>(&Vs[v_at(16 * q + srow, cch)]) = vst[q];
        }
    };

    // running max of row n (log2 units, the same in the row's four lanes) and
    // this lane's share of the row's sum (reduced over the lanes at the end)
    float m[TPW], l[TPW];
    f32x4 ot[TPW][8];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        m[tt] = -INFINITY;
        l[tt] = 0.f;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) ot[tt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // A row's zero weights still meet every staged value row inside the value
    // product, so a non-finite value of a node the row does not see (NaN or
    // Inf in another branch) would reach it as 0 * Inf.  A branch sees only
    // its ancestors (TreeWY, "Method"), so the draft nodes' block is staged
    // with non-finite values replaced by 0 (select), and vnf_all[tid] records
    // which of this thread's 32 staged values were (bit 8 q + 2 e + half).  If
    // any was (rare), each output column whose visible nodes include one that
    // carried a non-finite value in that column is set to NaN at the end.
    // Finite values: the same products as without the check.
    // zero the non-finite halves of v (chunk q of this thread's rows) and
    // record them in vnf
    auto scrub = [&](u32x4 &v, int q, uint32_t &vnf) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t x = v[e];
            const bool blo = (x & 0x7f80u) == 0x7f80u, bhi = (x & 0x7f800000u) == 0x7f800000u;
            vnf |= (blo ? 1u : 0u) << (8 * q + 2 * e);
            vnf |= (bhi ? 1u : 0u) << (8 * q + 2 * e + 1);
            v[e] = x & (blo ? 0xffff0000u : 0xffffffffu) & (bhi ? 0x0000ffffu : 0xffffffffu);
        }
    };
    if constexpr (DMA) issue_block(0, Ks, Vs);
    else load_block(0);
    for (int blk = 0; blk < nblk; ++blk) {
        // With direct loads the two buffers are separate LDS arrays chosen by
        // the block's parity (even blocks in Ks / Vs, odd ones in Ks2 / Vs2),
        // so that the compiler can tell this block's reads from the next
        // block's loads and does not wait for those loads before them (the
        // wait at the top of the next block covers them).
        const bool odd = DMA && (blk & 1);
        uint16_t *Kb = odd ? Ks2 : Ks, *Vb = odd ? Vs2 : Vs;
        if constexpr (DMA) {
            __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads of the block have landed
            lds_barrier();                   // everyone's have, and every wave is done with the other buffer
            if (blk >= nctx) {   // the draft nodes' block (the last one; workgroup-uniform): scrub in LDS
                uint32_t vnf = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x4 *p = reinterpret_cast<u32x4 *>(&Vb[v_at(16 * q + srow, cch)]);
                    u32x4 v = *p;
                    scrub(v, q, vnf);
                    *p = v;
                }
                vnf_all[tid] = vnf;
                lds_barrier();
            }
            if (blk + 1 < nblk) issue_block(blk + 1, odd ? Ks : Ks2, odd ? Vs : Vs2);
        } else {
            if (blk > 0) lds_barrier();   // every wave is done with the previous block
            if (blk >= nctx) {   // the draft nodes' block (the last one; workgroup-uniform)
                uint32_t vnf = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) scrub(vst[q], q, vnf);
                vnf_all[tid] = vnf;
            }
            store_block();
            lds_barrier();
            if (blk + 1 < nblk) load_block(blk + 1);
        }
        if (!active) continue;
        const bool nodeb = blk >= nctx;
        const int rem = k1 - (k0 + KB * blk);   // context keys left from this block on

        // scores S^T for keys 16 kt + 4 grp + i of row n (raw q.k); each K
        // fragment serves every tile of the wave; fragments of step
        // j = 4 kt + s are read KPF steps ahead
        f32x4 sc[TPW][NKT];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) sc[tt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // two fragments ahead: deeper prefetch spilled registers (4 ahead for K
        // and V: 8 spills, 676 vs 656 us on the batch-256 trees)
        constexpr int KPF = 2;
        u32x4 kf[KPF];
        auto kload = [&](int j) {   // row 16 (kt_lo + kt) + n, chunk 4 s + grp
            kf[j % KPF] = *reinterpret_cast<const u32x4 *>(&Kb[k_at(16 * (kt_lo + (j >> 2)) + n, 4 * (j & 3) + grp)]);
        };
#pragma unroll
        for (int j = 0; j < KPF; ++j) kload(j);
#pragma unroll
        for (int j = 0; j < 4 * NKT; ++j) {
            const u32x4 k = kf[j % KPF];
            if (j + KPF < 4 * NKT) kload(j + KPF);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
                sc[tt][j >> 2] = mfma(k, qf[tt][j & 3], sc[tt][j >> 2]);
        }

        // softmax per tile; P in bf16 hi + lo as the B operand of the value product
        u32x4 phi[TPW][NKS], plo[TPW][NKS];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            float x[NKT][4];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[kt][i] = sc[tt][kt][i];
            if (nodeb || rem < KB) {   // the last context block and the nodes' block: hide keys row n may not see
                const uint64_t vis = nodeb ? ancestry(tt) : ((1ull << rem) - 1ull);
                // bit 16 kt + i: key 16 (kt_lo + kt) + 4 grp + i
                const uint64_t vl = vis >> (4 * grp + 16 * kt_lo);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!((vl >> (16 * kt + i)) & 1ull)) x[kt][i] = -INFINITY;
            }
            float mloc = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, x[kt][i]);
            mloc *= a.scale_log2;   // the scale is positive: max commutes with it
            if (__ballot(mloc > m[tt] + RESCALE)) {   // some row grew past the margin: exact row max
                float mb = fmaxf(mloc, __shfl_xor(mloc, 16));
                mb = fmaxf(mb, __shfl_xor(mb, 32));
                const float mnew = fmaxf(m[tt], mb);
                const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[tt] - mnew);
                l[tt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ot[tt][mt][i] *= alpha;
                m[tt] = mnew;
            }
            const float mneg = m[tt] == -INFINITY ? 0.f : -m[tt];   // nothing visible yet: p = 0
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[kt][i] = __builtin_amdgcn_exp2f(fmaf(x[kt][i], a.scale_log2, mneg));
                    l[tt] += x[kt][i];
                }
            if constexpr (NKT == 1) {
                // one 16-key tile: the lower (even tile) or upper (odd tile)
                // half of its 32-key value step; the other half of P is 0
                uint32_t h0, l0, h1, l1;
                split_bf16x2(x[0][0], x[0][1], h0, l0);
                split_bf16x2(x[0][2], x[0][3], h1, l1);
                const bool upper = kt_lo & 1;
                phi[tt][0] = upper ? u32x4{0u, 0u, h0, h1} : u32x4{h0, h1, 0u, 0u};
                plo[tt][0] = upper ? u32x4{0u, 0u, l0, l1} : u32x4{l0, l1, 0u, 0u};
            } else {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
                    split_bf16x2(x[2 * ks][0], x[2 * ks][1], h0, l0);
                    split_bf16x2(x[2 * ks][2], x[2 * ks][3], h1, l1);
                    split_bf16x2(x[2 * ks + 1][0], x[2 * ks + 1][1], h2, l2);
                    split_bf16x2(x[2 * ks + 1][2], x[2 * ks + 1][3], h3, l3);
                    phi[tt][ks] = u32x4{h0, h1, h2, h3};
                    plo[tt][ks] = u32x4{l0, l1, l2, l3};
                }
            }
        }

        // O^T += V^T P^T over the block's two 32-key steps; each V^T fragment
        // serves every tile; fragments of step j = 8 ks + mt are read PF
        // steps ahead of their MFMAs
        constexpr int PF = 2;
        u32x4 vf[PF];
        // lane s = n of group grp addresses key 32 ks + 16 h + 4 grp + s / 4,
        // columns 16 mt + 4 (s % 4) .. +3, and receives column 16 mt + n of
        // keys 32 ks + 16 h + 4 grp + e, e = 0..3 (k-slots 4h .. 4h+3)
        const int vsub = 4 * (n & 1);   // element offset inside the 16-byte chunk
        auto vload = [&](int j) {
            const int ks = (kt_lo >> 1) + (j >> 3), mt = j & 7;
            const int c = 2 * mt + ((n & 3) >> 1);
            const int r0 = 32 * ks + 4 * grp + (n >> 2);
            const u32x2 va = lds_read_tr16(&Vb[v_at(r0, c) + vsub]);
            const u32x2 vb = lds_read_tr16(&Vb[v_at(r0 + 16, c) + vsub]);
            vf[j % PF] = u32x4{va.x, va.y, vb.x, vb.y};
        };
#pragma unroll
        for (int j = 0; j < PF; ++j) vload(j);
#pragma unroll
        for (int j = 0; j < 8 * NKS; ++j) {
            const u32x4 v = vf[j % PF];
            if (j + PF < 8 * NKS) vload(j + PF);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                ot[tt][j & 7] = mfma(v, phi[tt][j >> 3], ot[tt][j & 7]);
                ot[tt][j & 7] = mfma(v, plo[tt][j >> 3], ot[tt][j & 7]);
            }
        }
    }
    // did any staged node value turn out non-finite? (vnf words of all threads,
    // visible since the node block's barrier; four per lane, one ballot)
    bool vpoison = false;
    if (nctx < nblk) {
        const u32x4 f = *reinterpret_cast<const u32x4 *>(&vnf_all[4 * lane]);
        vpoison = __ballot((f[0] | f[1] | f[2] | f[3]) != 0u) != 0ull;
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        l[tt] += __shfl_xor(l[tt], 16);
        l[tt] += __shfl_xor(l[tt], 32);
    }
    if constexpr (KG > 1) {
        // key groups 1 .. KG-1 of each tile leave (O, max, sum) in the LDS block
        // (slot p = tile (KG - 1) + group - 1: 2048 floats of O laid out
        // [mt][lane][4], then 128 floats of (max, sum) per slot after the
        // third slot); group 0 merges them and writes the tile
        lds_barrier();   // every wave is done with the last block
        float *ob = reinterpret_cast<float *>(Ks);   // slots 0, 1
        float *vb = reinterpret_cast<float *>(Vs);   // slot 2, then the (max, sum) pairs
        auto slot_o = [&](int p) { return p < 2 ? ob + 2048 * p : vb; };
        float2 *ml = reinterpret_cast<float2 *>(vb + 2048);
        if (kg > 0) {
            const int p = wr * (KG - 1) + kg - 1;
            float *o = slot_o(p);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                *reinterpret_cast<f32x4 *>(o + (mt * 64 + lane) * 4) = ot[0][mt];
            ml[p * 64 + lane] = make_float2(m[0], l[0]);
        }
        lds_barrier();
        if (kg == 0) {
            float mm = m[0];
#pragma unroll
            for (int q = 1; q < KG; ++q) mm = fmaxf(mm, ml[(wr * (KG - 1) + q - 1) * 64 + lane].x);
            const float fs = m[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[0] - mm);
            l[0] *= fs;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) ot[0][mt] *= fs;
#pragma unroll
            for (int q = 1; q < KG; ++q) {
                const int p = wr * (KG - 1) + q - 1;
                const float2 pml = ml[p * 64 + lane];
                const float f = pml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pml.x - mm);
                l[0] += f * pml.y;
                const float *o = slot_o(p);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    const f32x4 po = *reinterpret_cast<const f32x4 *>(o + (mt * 64 + lane) * 4);
                    ot[0][mt] += f * po;
                }
            }
            m[0] = mm;
        } else {
            rvalid[0] = false;   // group 0 writes the tile
        }
    }

    // lane (n, grp) holds columns 16 mt + 4 grp .. +3 of its rows
    if (vpoison) {   // rare: column c of a row turns NaN if a node it sees had a non-finite value there
        const float qnan = __int_as_float(0x7fc00000);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            uint32_t pm = 0;   // bit 4 mt + i: column 16 mt + 4 grp + i
#pragma unroll 1
            for (int x = 0; x < 32; ++x) {
                const int col = 16 * (x >> 2) + 4 * grp + (x & 3);
                for (uint64_t m = ancestry(tt); m; m &= m - 1) {
                    const int j = __builtin_ctzll(m);   // node row j was staged by thread 16 (j % 16) + col / 8
                    if ((vnf_all[16 * (j & 15) + (col >> 3)] >> (8 * (j >> 4) + (col & 7))) & 1u) pm |= 1u << x;
                }
            }
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if ((pm >> (4 * mt + i)) & 1u) ot[tt][mt][i] = qnan;
        }
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        if (!rvalid[tt]) continue;
        if (a.n_split == 1) {
            int tr, gr;
            row_index(tt, tr, gr);
            const size_t orow = (size_t)(lo + tr) * a.Hq + hk * G + gr;
            const float inv = 1.f / l[tt];
            float *op = a.out + orow * D + 4 * grp;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                *reinterpret_cast<float4 *>(op + 16 * mt) = make_float4(ot[tt][mt][0] * inv, ot[tt][mt][1] * inv,
                                                                        ot[tt][mt][2] * inv, ot[tt][mt][3] * inv);
            if (grp == 0 && a.lse) a.lse[orow] = (m[tt] + log2f(l[tt])) * LN2;
        } else {
            float *rec = a.ws + ATTN_WS_HEADER_BYTES / 4 +
                         ((((size_t)b * a.Hkv + hk) * a.n_split + sp) * a.n_rg + rg) * part_floats(RROWS);
            const int rl = 16 * (TPW * wr + tt) + n;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                *reinterpret_cast<float4 *>(rec + rl * D + 16 * mt + 4 * grp) =
                    make_float4(ot[tt][mt][0], ot[tt][mt][1], ot[tt][mt][2], ot[tt][mt][3]);
            if (grp == 0) {
                rec[RROWS * D + rl] = m[tt];
                rec[RROWS * D + RROWS + rl] = l[tt];
            }
        }
    }
}

// One workgroup per unit: unit = ((b Hkv + hk) n_split + sp) n_rg + rg, the
// row groups of one (request, kv-head, part) neighbours on one XCD.
template <int TPW>
__global__ __launch_bounds__(AT) __attribute__((amdgpu_waves_per_eu(TPW == 1 ? 3 : 2))) void attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KB * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[KB * D];
    __shared__ __attribute__((aligned(16))) uint32_t vnf_all[AT];   // non-finite node values, per thread
    const int n_units = a.B * a.Hkv * a.n_split * a.n_rg;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int rg = unit % a.n_rg;
    int rest = unit / a.n_rg;
    const int sp = rest % a.n_split;
    rest /= a.n_split;
    attn_unit<TPW>(a, rest / a.Hkv, rest % a.Hkv, sp, rg, unit, Ks, Vs, Ks, Vs, vnf_all);
}

// ---- scheduled launch: a resident grid working through a sorted unit list ----
// Units differ several-fold in length (context length, row groups), and
// workgroups are dispatched in order, so a grid of one workgroup per unit
// leaves compute units idle behind long units.  Instead a grid that fits on
// the chip at once works through one list of the units that do work, sorted
// by length (longest first; every workgroup builds the same list in LDS).
// The list is cut into chunks of 64 positions dealt boustrophedon to eight
// sub-lists (chunk i to sub-list i % 16 or 15 - i % 16), and the workgroups
// with blockIdx % 8 = x (one XCD under round-robin dispatch) take positions of
// sub-list x from a counter in the workspace, longest first, as they become
// free: the deal balances the sub-lists, the counter absorbs the workgroups'
// differing speeds, and neighbouring positions (the row groups of one request
// and kv-head) run on one XCD at the same time and share its L2.
constexpr int SCHED_ITEMS = ATTN_SCHED_ITEMS;   // (request, context part) items the list can hold
constexpr int SCHED_BUCKETS = 64;    // length classes of the counting sort

struct AttnSched {
    int item[SCHED_ITEMS];        // scheduled items in list order: item | row groups << 16
    int first[SCHED_ITEMS + 1];   // list position of each scheduled item's first unit
    int info[SCHED_ITEMS];        // per item: units | row groups << 12 | bucket << 20
    int base[SCHED_BUCKETS + 1];  // bucket starts, then running positions
    int n_live;
};

// Units of item (request b, context part sp), their row groups, and the
// item's length (blocks it streams).  Parts that do nothing contribute no
// unit; a request with bad offsets or no rows keeps one unit for its status.
__device__ __forceinline__ void sched_item(const AttnArgs &a, int b, int sp, int &cnt, int &nrg, int &len) {
    int lo, N, c0, Lc;
    const int st = attn_request(a, b, lo, N, c0, Lc);
    cnt = 0;
    nrg = 0;
    len = 0;
    if (st == GDN_TREE_S_BAD_OFFSETS || N == 0) {
        cnt = sp == 0 ? 1 : 0;
        return;
    }
    if (sp > 0 && (st != GDN_TREE_S_OK || sp * a.split >= Lc)) return;
    nrg = min(a.n_rg, (N * a.G + a.rows_wg - 1) / a.rows_wg);
    cnt = a.Hkv * nrg;
    if (st == GDN_TREE_S_OK) {
        const int k0 = sp * a.split, k1 = min(Lc, k0 + a.split);
        len = (k1 > k0 ? (k1 - k0 + KB - 1) / KB : 0) + (sp == 0 ? 1 : 0);
    }
}

// Lanes of the wave whose b-bit value v equals this lane's (nbits ballots).
__device__ __forceinline__ uint64_t same_value(int v, int nbits) {
    uint64_t eq = __ballot(1);
    for (int bit = 0; bit < nbits; ++bit) {
        const uint64_t bal = __ballot((v >> bit) & 1);
        eq &= ((v >> bit) & 1) ? bal : ~bal;
    }
    return eq;
}

// Wave 0 builds the list: a stable counting sort of the items by length class
// (longest first), then the prefix of their unit counts.
__device__ void build_sched(const AttnArgs &a, AttnSched &sc) {
    const int lane = threadIdx.x & 63;
    const int n_items = a.B * a.n_split;
    const int lmax = (min(a.split, a.max_ctx) + KB - 1) / KB + 1;
    int shift = 0;
    while ((lmax >> shift) >= SCHED_BUCKETS) ++shift;
    const uint64_t below = (1ull << lane) - 1ull;
    sc.base[lane] = 0;
    if (lane == 0) sc.base[SCHED_BUCKETS] = 0;
    for (int i0 = 0; i0 < n_items; i0 += 64) {   // classes and counts
        const int i = i0 + lane;
        int cnt = 0, nrg = 0, len = 0;
        if (i < n_items) sched_item(a, i / a.n_split, i % a.n_split, cnt, nrg, len);
        const int bk = cnt > 0 ? SCHED_BUCKETS - 1 - min(len >> shift, SCHED_BUCKETS - 1) : SCHED_BUCKETS;
        if (i < n_items) sc.info[i] = cnt | (nrg << 12) | (bk << 20);
        const uint64_t eq = same_value(bk, 7);
        if ((eq & below) == 0ull && bk < SCHED_BUCKETS) sc.base[bk] += __popcll(eq);
    }
    int c = sc.base[lane];   // exclusive scan of the 64 class counts
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int up = __shfl_up(incl, off);
        if (lane >= off) incl += up;
    }
    sc.base[lane] = incl - c;
    if (lane == 63) sc.n_live = incl;
    for (int i0 = 0; i0 < n_items; i0 += 64) {   // stable scatter
        const int i = i0 + lane;
        const int inf = i < n_items ? sc.info[i] : (SCHED_BUCKETS << 20);
        const int bk = inf >> 20;
        const uint64_t eq = same_value(bk, 7);
        if (bk < SCHED_BUCKETS) {
            const int pos = sc.base[bk] + __popcll(eq & below);
            sc.item[pos] = i | (((inf >> 12) & 0xff) << 16);
            sc.first[pos] = inf & 0xfff;   // unit count for now
        }
        if ((eq & below) == 0ull && bk < SCHED_BUCKETS) sc.base[bk] += __popcll(eq);
    }
    const int n_live = sc.n_live;
    int carry = 0;   // unit counts -> exclusive prefix
    for (int p0 = 0; p0 < n_live; p0 += 64) {
        const int p = p0 + lane;
        const int v = p < n_live ? sc.first[p] : 0;
        int incl2 = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int up = __shfl_up(incl2, off);
            if (lane >= off) incl2 += up;
        }
        if (p < n_live) sc.first[p] = carry + incl2 - v;
        carry += __shfl(incl2, 63);
    }
    if (lane == 0) sc.first[n_live] = carry;
}

template <int TPW>
__global__ __launch_bounds__(AT) __attribute__((amdgpu_waves_per_eu(TPW == 1 ? 3 : 2))) void attn_sched_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KB * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[KB * D];
    // 128-row units stage two blocks (direct loads into one while the other is computed)
    __shared__ __attribute__((aligned(16))) uint16_t Ks2[TPW == 2 ? KB * D : 8];
    __shared__ __attribute__((aligned(16))) uint16_t Vs2[TPW == 2 ? KB * D : 8];
    __shared__ __attribute__((aligned(16))) uint32_t vnf_all[AT];   // non-finite node values, per thread
    __shared__ AttnSched sc;
    if ((threadIdx.x >> 6) == 0) build_sched(a, sc);
    lds_barrier();
    __shared__ int ticket;
    const int n_live = sc.n_live, total = sc.first[n_live];
    const int x = blockIdx.x & 7;   // sub-list
    int *counter = reinterpret_cast<int *>(a.ws) + x;
    for (;;) {
        if (threadIdx.x == 0) ticket = atomicAdd(counter, 1);
        lds_barrier();
        const int tk = ticket, chunk = tk >> 6;   // chunk-th chunk of sub-list x
        const int k = 64 * (16 * (chunk >> 1) + ((chunk & 1) ? 15 - x : x)) + (tk & 63);
        if (k >= total) break;
        int lo = 0, hi = n_live - 1;   // the scheduled item holding position k
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sc.first[mid] <= k) lo = mid;
            else hi = mid - 1;
        }
        const int it = sc.item[lo] & 0xffff, nrg = sc.item[lo] >> 16, j = k - sc.first[lo];
        const int b = it / a.n_split, sp = it - b * a.n_split;
        const int hk = nrg > 0 ? j / nrg : 0, rg = nrg > 0 ? j - hk * nrg : 0;
        attn_unit<TPW>(a, b, hk, sp, rg, k, Ks, Vs, Ks2, Vs2, vnf_all);
        lds_barrier();   // every wave is done with the LDS block (and the ticket) before the next unit
    }
}

// Zero the scheduling counters before a scheduled launch (a kernel rather than
// a memset, so that the pair can be captured in a graph).
__global__ void attn_reset_kernel(float *ws) {
    if (threadIdx.x < 8) reinterpret_cast<int *>(ws)[threadIdx.x] = 0;
}


// Merge the context parts of each row: thread (row, quarter) owns 32 columns.
// MAXP > 0: at most MAXP parts, every part's loads issued together; MAXP = 0:
// any number of parts, one after another.
template <int MAXP>
__global__ __launch_bounds__(AT) void attn_merge_kernel(AttnArgs a) {
    const int unit = blockIdx.x;
    const int rg = unit % a.n_rg;
    const int rest = unit / a.n_rg;
    const int hk = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const int tid = threadIdx.x;
    int lo, N, c0, Lc;
    int st = attn_request(a, b, lo, N, c0, Lc);
    if (st == GDN_TREE_S_BAD_OFFSETS) return;
    const int G = a.G;
    const int R = N * G;
    const int ROWS = a.rows_wg;
    if (ROWS * rg >= R) return;   // a row group past the request's rows (decided before the mask vote)
    st = check_masks(a, st, lo, N);
    if (st != GDN_TREE_S_OK) {
        nan_rows(a, lo, hk, ROWS * rg, nan_end(a, rg, R));
        return;
    }
    const size_t PART = part_floats(ROWS);
    const int nparts = Lc > 0 ? (Lc + a.split - 1) / a.split : 1;
    const size_t stride = (size_t)a.n_rg * PART;   // between consecutive parts
    const float *rec = a.ws + ATTN_WS_HEADER_BYTES / 4 + (((size_t)b * a.Hkv + hk) * a.n_split * a.n_rg + rg) * PART;
    if constexpr (MAXP > 0) {
        // thread (row, slice): 8 threads per row, 16 columns each; every part's
        // max, sum and slice are requested before any of them is used
        const int sl = tid & 7;
        for (int rl = tid >> 3; rl < ROWS; rl += AT / 8) {
            const int r = ROWS * rg + rl;
            if (r >= R) break;
            const int t = r / G, g = r - t * G;
            const size_t orow = (size_t)(lo + t) * a.Hq + hk * G + g;
            float mp[MAXP], lp[MAXP];
            f32x4 ov[MAXP][4];
#pragma unroll
            for (int s = 0; s < MAXP; ++s) {   // reads stay inside the request's parts (index clamped)
                const size_t sp = (size_t)min(s, nparts - 1) * stride;
                mp[s] = rec[sp + ROWS * D + rl];
                lp[s] = rec[sp + ROWS * D + ROWS + rl];
                const f32x4 *src = reinterpret_cast<const f32x4 *>(rec + sp + rl * D + 16 * sl);
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[s][i] = src[i];
            }
            float M = -INFINITY, L = 0.f;
#pragma unroll
            for (int s = 0; s < MAXP; ++s)
                if (s < nparts) M = fmaxf(M, mp[s]);
            f32x4 acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < MAXP; ++s) {
                if (s < nparts) {
                    const float wgt = __builtin_amdgcn_exp2f(mp[s] - M);
                    L += wgt * lp[s];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] += wgt * ov[s][i];
                }
            }
            const float inv = 1.f / L;
            float *op = a.out + orow * D + 16 * sl;
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4 *>(op + 4 * i) = acc[i] * inv;
            if (sl == 0 && a.lse) a.lse[orow] = (M + log2f(L)) * LN2;
        }
    } else {
        const int quarter = tid & 3;
        for (int rl = tid >> 2; rl < ROWS; rl += AT / 4) {
            const int r = ROWS * rg + rl;
            if (r >= R) break;
            const int t = r / G, g = r - t * G;
            const size_t orow = (size_t)(lo + t) * a.Hq + hk * G + g;
            float *op = a.out + orow * D + 32 * quarter;
            float M = -INFINITY, L = 0.f;
            f32x4 acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < nparts; ++s) M = fmaxf(M, rec[s * stride + ROWS * D + rl]);
            for (int s = 0; s < nparts; ++s) {
                const float *rs = rec + s * stride;
                const float wgt = __builtin_amdgcn_exp2f(rs[ROWS * D + rl] - M);
                L += wgt * rs[ROWS * D + ROWS + rl];
                const f32x4 *src = reinterpret_cast<const f32x4 *>(rs + rl * D + 32 * quarter);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += wgt * src[i];
            }
            const float inv = 1.f / L;
#pragma unroll
            for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4 *>(op + 4 * i) = acc[i] * inv;
            if (quarter == 0 && a.lse) a.lse[orow] = (M + log2f(L)) * LN2;
        }
    }
}

}  // namespace

hipError_t launch_ancestry(const Args &a, hipStream_t stream) {
    ancestry_kernel<<<dim3((a.B + 3) / 4), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

namespace {
constexpr int MAX_DEVICES = 64;
// Launch facts of the current device, cached per device: its compute units and
// the scheduled attention kernel's resident workgroups per CU (0 = unknown).
// Threads that race to fill an entry compute the same value; the atomics keep
// those stores and loads well defined.
std::atomic<int> g_cus[MAX_DEVICES];
std::atomic<int> g_occupancy[MAX_DEVICES], g_occupancy2[MAX_DEVICES];

int cached_fact(std::atomic<int> *table, int dev, int (*query)(int)) {
    if (dev < 0 || dev >= MAX_DEVICES) return query(dev);
    int v = table[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        v = query(dev);
        if (v > 0) table[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

int query_cus(int dev) {
    int cus = 0;
    return hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? cus : 0;
}

template <int TPW>
int query_occupancy(int) {
    int occ = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, attn_sched_kernel<TPW>, AT, 0) == hipSuccess ? occ : 0;
}

// Resident workgroups of the scheduled launch (TPW tiles per wave) on the
// current device: the runtime's occupancy (registers and LDS) times the CUs.
template <int TPW>
int resident_workgroups() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    return cached_fact(TPW == 1 ? g_occupancy : g_occupancy2, dev, query_occupancy<TPW>) *
           cached_fact(g_cus, dev, query_cus);
}
}  // namespace

// ---- the workspace of the allocation-free entry point ------------------------
// A file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  On the host the array's name is only a stand-in, not
// a device address, so no host code passes it to a kernel or a copy: the first
// call on each device looks up that device's copy with hipGetSymbolAddress
// (with the device current) and keeps the address per device.
static __device__ __align__(256) unsigned char scratch[GDN_TREE_STATIC_SCRATCH_BYTES];

namespace {
std::atomic<void *> g_scratch[MAX_DEVICES];
}  // namespace

hipError_t static_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t stream) {
    const int units = a.B * a.Hkv * a.n_split * a.n_rg;
    if (a.rows_wg == 128) {
        // the host chose 128-row units only where the scheduled launch takes the batch
        const int resident = (resident_workgroups<2>() / 8) * 8;
        if (resident < 8 || (long long)a.B * a.n_split > SCHED_ITEMS || a.n_rg >= 256 || a.Hkv * a.n_rg >= 4096)
            return hipErrorInvalidValue;
        attn_reset_kernel<<<dim3(1), dim3(64), 0, stream>>>(a.ws);
        attn_sched_kernel<2><<<dim3(min(resident, xcd_grid(units))), dim3(AT), 0, stream>>>(a);
    } else {
        if (a.rows_wg != 64) return hipErrorInvalidValue;
        const int resident = (resident_workgroups<1>() / 8) * 8;
        // the list packs row groups in 8 bits and an item's unit count in 12
        const bool sched = resident >= 8 && (long long)a.B * a.n_split <= SCHED_ITEMS && a.n_rg < 256 &&
                           a.Hkv * a.n_rg < 4096;
        if (sched) {
            attn_reset_kernel<<<dim3(1), dim3(64), 0, stream>>>(a.ws);
            attn_sched_kernel<1><<<dim3(min(resident, xcd_grid(units))), dim3(AT), 0, stream>>>(a);
        } else {
            attn_kernel<1><<<dim3(xcd_grid(units)), dim3(AT), 0, stream>>>(a);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    if (a.n_split <= 4)
        attn_merge_kernel<4><<<dim3(a.B * a.Hkv * a.n_rg), dim3(AT), 0, stream>>>(a);
    else
        attn_merge_kernel<0><<<dim3(a.B * a.Hkv * a.n_rg), dim3(AT), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
