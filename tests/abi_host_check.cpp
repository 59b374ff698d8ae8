// Host-side argument checks of every C-ABI entry point, for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code
// (tests/test_abi_sanitized.py builds and runs it).  Every call below is
// rejected on the host (or is a no-op batch), so no GPU is touched.  Exit
// status = number of failed checks.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn_tree.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
    if (got != want) {
        printf("FAIL %s: got %d want %d\n", what, got, want);
        ++failures;
    }
}

int main() {
    // aligned, never dereferenced: every call fails before a launch
    alignas(16) static unsigned char arena[4 << 20];
    void *P = arena;
    const float *F = reinterpret_cast<const float *>(arena);
    float *Fw = reinterpret_cast<float *>(arena);
    const uint16_t *H = reinterpret_cast<const uint16_t *>(arena);
    const int32_t *I = reinterpret_cast<const int32_t *>(arena);
    int32_t *Iw = reinterpret_cast<int32_t *>(arena);
    uint64_t *M = reinterpret_cast<uint64_t *>(arena);
    const float *Fmis = reinterpret_cast<const float *>(arena + 4);
    float *Fw2 = reinterpret_cast<float *>(arena + (1 << 20));   // regions 1 MiB apart: no overlap
    float *Fw3 = reinterpret_cast<float *>(arena + (2 << 20));

    gdn_tree_dims d = {4, 32, 16, 128, 128, 20, 8, 4};
    gdn_tree_dims bad = d;
    bad.Hk = 3;
    gdn_tree_dims hd = d;
    hd.d_k = 64;
    gdn_tree_dims mn = d;
    mn.max_nodes = 65;
    gdn_tree_dims empty = d;
    empty.B = 0;
    empty.T = 0;

    expect("verify null dims", gdn_tree_verify(nullptr, F, I, H, H, H, F, F, I, I, Fw, Fw, M, Iw, nullptr), GDN_TREE_E_NULL);
    expect("verify bad Hk", gdn_tree_verify(&bad, F, I, H, H, H, F, F, I, I, Fw, Fw, M, Iw, nullptr), GDN_TREE_E_DIMS);
    expect("verify head dim", gdn_tree_verify(&hd, F, I, H, H, H, F, F, I, I, Fw, Fw, M, Iw, nullptr), GDN_TREE_E_HEAD_DIM);
    expect("verify max nodes", gdn_tree_verify(&mn, F, I, H, H, H, F, F, I, I, Fw, Fw, M, Iw, nullptr), GDN_TREE_E_MAX_NODES);
    expect("verify null S0", gdn_tree_verify(&d, nullptr, I, H, H, H, F, F, I, I, Fw, Fw, M, Iw, nullptr), GDN_TREE_E_NULL);
    expect("verify misaligned", gdn_tree_verify(&d, Fmis, I, H, H, H, F, F, I, I, Fw, Fw, M, Iw, nullptr), GDN_TREE_E_ALIGN);
    expect("verify empty", gdn_tree_verify(&empty, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                           nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), GDN_TREE_OK);
    expect("commit null path", gdn_tree_commit(&d, F, Fw, I, F, H, F, I, I, nullptr, I, Iw, nullptr), GDN_TREE_E_NULL);
    expect("commit bad dims", gdn_tree_commit(&bad, F, Fw, I, F, H, F, I, I, I, I, Iw, nullptr), GDN_TREE_E_DIMS);
    expect("replay misaligned", gdn_tree_commit_replay(&d, Fmis, Fw, I, H, H, F, F, I, I, I, I, Iw, nullptr), GDN_TREE_E_ALIGN);
    expect("accepted_path null", gdn_tree_accepted_path(&d, I, I, nullptr, Iw, Iw, Iw, nullptr), GDN_TREE_E_NULL);
    expect("accept_greedy null", gdn_tree_accept_greedy(&d, I, I, I, I, nullptr, Iw, Iw, Iw, Iw, nullptr), GDN_TREE_E_NULL);
    expect("accept_commit bad", gdn_tree_accept_commit(&mn, F, Fw, I, F, H, F, I, I, I, I, I, Iw, Iw, Iw, Iw, nullptr),
           GDN_TREE_E_MAX_NODES);
    expect("commit_node null accept", gdn_tree_commit_node(&d, F, Fw, I, F, H, F, I, I, nullptr, Iw, Iw, Iw, nullptr),
           GDN_TREE_E_NULL);
    gdn_tree_dims d2 = d;
    d2.Hv = 16;
    expect("commit_verify mismatched", gdn_tree_commit_verify(&d2, &d, F, Fw, I, F, H, F, I, I, I, Iw, Iw, Iw, H, H, H,
                                                              F, F, I, I, Fw, Fw, M, Iw, nullptr), GDN_TREE_E_DIMS);
    expect("commit_verify overlap", gdn_tree_commit_verify(&d, &d, F, Fw, I, F, H, F, I, I, I, Iw, Iw, Iw, H, H, H, F,
                                                           F, I, I, Fw, Fw, M, Iw, nullptr), GDN_TREE_E_OVERLAP);
    expect("accept_commit_verify null", gdn_tree_accept_commit_verify(&d, &d, F, Fw, I, F, H, F, I, I, I, I, nullptr, Iw,
                                                                      Iw, Iw, Iw, H, H, H, F, F, I, I, Fw2,
                                                                      Fw3, M, Iw, nullptr),
           GDN_TREE_E_NULL);
    gdn_tree_dims big = d;
    big.T = 1 << 24;
    expect("budget too many nodes", gdn_tree_budget_select(&big, I, I, F, 10, 0.f, Fw, reinterpret_cast<uint8_t *>(P),
                                                           Iw, Iw, nullptr), GDN_TREE_E_SIZE);
    expect("ancestry null", gdn_tree_ancestry(&d, nullptr, I, M, Iw, nullptr), GDN_TREE_E_NULL);
    expect("storeall verify null", gdn_tree_verify_storeall(&d, F, I, H, H, H, F, F, I, I, Fw, nullptr, Iw, nullptr),
           GDN_TREE_E_NULL);
    expect("storeall commit misaligned", gdn_tree_commit_storeall(&d, Fmis, Fw, I, F, I, I, I, Iw, nullptr),
           GDN_TREE_E_ALIGN);

    gdn_tree_attn_dims ad = {4, 8, 2, 128, 10, 100, 8, 50, 50};
    gdn_tree_attn_dims abad = ad;
    abad.Hkv = 3;
    expect("attention bad dims", gdn_tree_attention(&abad, H, H, H, I, H, H, I, M, 0.1f, Fw, Fw, P, 4096, Iw, nullptr),
           GDN_TREE_E_DIMS);
    expect("attention bad scale", gdn_tree_attention(&ad, H, H, H, I, H, H, I, M, -1.f, Fw, Fw, P, 4096, Iw, nullptr),
           GDN_TREE_E_DIMS);
    expect("attention small workspace", gdn_tree_attention(&ad, H, H, H, I, H, H, I, M, 0.1f, Fw, Fw, P, 16, Iw, nullptr),
           GDN_TREE_E_WORKSPACE);
    gdn_tree_attn_dims asplit = {256, 32, 8, 128, 512, 4096, 4, 1024, 256};
    expect("attention static beyond scratch", gdn_tree_attention_static(&asplit, H, H, H, I, H, H, I, M, 0.1f, Fw, Fw,
                                                                        Iw, nullptr), GDN_TREE_E_SCRATCH);
    expect("attention static null", gdn_tree_attention_static(&ad, nullptr, H, H, I, H, H, I, M, 0.1f, Fw, Fw, Iw,
                                                               nullptr), GDN_TREE_E_NULL);
    if (gdn_tree_attention_workspace_bytes(&ad) != 256) {
        printf("FAIL workspace bytes\n");
        ++failures;
    }
    if (gdn_tree_attention_workspace_bytes(&asplit) <= GDN_TREE_STATIC_SCRATCH_BYTES) {
        printf("FAIL split workspace\n");
        ++failures;
    }
    if (gdn_tree_state_bytes(&d, 1) != (size_t)20 * 32 * 128 * 128 * 4 || gdn_tree_state_bytes(&bad, 0) != 0) {
        printf("FAIL state bytes\n");
        ++failures;
    }
    for (int c = -12; c < 12; ++c) {
        const char *s = gdn_tree_strerror(c);
        if (!s || !strlen(s)) {
            printf("FAIL strerror %d\n", c);
            ++failures;
        }
    }
    if (gdn_tree_abi_version() != GDN_TREE_ABI_VERSION) ++failures;
    printf("%d failures\n", failures);
    return failures;
}
