// Host-side entry points of libtokengate under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every call here either runs on the host only
// (kept counts, random budgets, status strings, workspace sizes) or must be
// refused by argument validation before any HIP call (fake device pointers
// that are never dereferenced), so no GPU is needed.  Exit status 0 when every
// call returns its documented status; a sanitizer report aborts.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "tokengate.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                               \
        }                                                             \
    } while (0)

int main() {
    // status strings
    for (int st = -1; st <= 5; ++st) EXPECT(tg_status_string(st) != nullptr && strlen(tg_status_string(st)) > 0);

    // kept counts on random spans and budgets (host arrays of exact sizes)
    std::mt19937 rng(7);
    for (int trial = 0; trial < 200; ++trial) {
        const int n_seqs = (int)(rng() % 9);
        std::vector<int32_t> cu(n_seqs + 1), b(n_seqs), e(n_seqs), k(n_seqs), ck(n_seqs + 1);
        for (int s = 0; s < n_seqs; ++s) {
            const int n = (int)(rng() % 5000);
            cu[s + 1] = cu[s] + n;
            b[s] = n ? (int)(rng() % (n + 1)) : 0;
            e[s] = b[s] + (n - b[s] ? (int)(rng() % (n - b[s] + 1)) : 0);
            k[s] = (int)(rng() % 6000);
        }
        EXPECT(tg_kept_counts(n_seqs, cu.data(), b.data(), e.data(), k.data(), ck.data()) == TG_OK);
        int64_t acc = 0;
        for (int s = 0; s < n_seqs; ++s) {
            const int64_t nd = e[s] - b[s];
            acc += (k[s] < nd ? k[s] : nd) + (cu[s + 1] - cu[s] - nd);
            EXPECT(ck[s + 1] == acc);
        }
        std::vector<int32_t> kb(n_seqs);
        EXPECT(tg_random_budgets(rng(), n_seqs, b.data(), e.data(), kb.data()) == TG_OK);
        for (int s = 0; s < n_seqs; ++s) EXPECT(kb[s] >= 0 && kb[s] <= e[s] - b[s]);
    }
    {
        int32_t cu[2] = {0, 10}, b[1] = {3}, e[1] = {2}, k[1] = {1}, ck[2];
        EXPECT(tg_kept_counts(1, cu, b, e, k, ck) == TG_ERR_INVALID_ARG);   // span end before begin
        EXPECT(tg_kept_counts(1, nullptr, b, e, k, ck) == TG_ERR_INVALID_ARG);
        EXPECT(tg_random_budgets(1, 1, b, e, k) == TG_ERR_INVALID_ARG);
    }

    // workspace sizes, including extreme arguments
    EXPECT(tg_topk_workspace_bytes(-1, 10, 10) == 0);
    EXPECT(tg_topk_workspace_bytes(8, 1 << 20, 1 << 20) > 0);
    EXPECT(tg_random_k_workspace_bytes(8, 1 << 20, 1 << 20) > tg_topk_workspace_bytes(8, 1 << 20, 1 << 20));
    EXPECT(tg_attn_workspace_bytes(4, 100000, 8, 128) > 0);
    EXPECT(tg_attn_decode_workspace_bytes(4, 100000, 16, 128) > 0);
    EXPECT(tg_attn_gate_grads_workspace_bytes(4, 100000, 40000, 16, 128) > 0);
    EXPECT(tg_topk_noalloc_max_bytes() > 0);

    // validation paths: refused before any HIP call
    const void* F = (const void*)(uintptr_t)0x1000;   // fake, 256-B aligned, never dereferenced
    const int32_t* FI = (const int32_t*)F;
    float* FF = (float*)(uintptr_t)0x1000;
    int32_t* FO = (int32_t*)(uintptr_t)0x1000;
    EXPECT(tg_gate_score(F, TG_BF16, 100, 100, 100, F, nullptr, (const float*)F, 0.0f, 256, FF, nullptr) ==
           TG_ERR_INVALID_ARG);                                                                  // d_model % 8
    EXPECT(tg_gate_score(F, 7, 100, 128, 128, F, nullptr, (const float*)F, 0.0f, 256, FF, nullptr) ==
           TG_ERR_INVALID_ARG);                                                                  // dtype
    EXPECT(tg_topk_select((const float*)F, 1, 100, 200, FI, FI, FI, FI, FI, FO, (void*)F, 1 << 20, nullptr) ==
           TG_ERR_INVALID_ARG);                                                                  // max_seqlen > total
    EXPECT(tg_topk_select((const float*)F, 1, 100, 100, FI, FI, FI, FI, FI, FO, (void*)F, 1, nullptr) ==
           TG_ERR_WORKSPACE);
    EXPECT(tg_topk_select_noalloc((const float*)F, 1, 1 << 22, 1 << 22, FI, FI, FI, FI, FI, FO, nullptr) ==
           TG_ERR_UNSUPPORTED);                                                                  // beyond its array
    EXPECT(tg_gather_kept(F, TG_BF16, 64, 64, nullptr, FI, 10, 1, FI, FI, nullptr, nullptr, FO, nullptr) ==
           TG_ERR_INVALID_ARG);                                                                  // no x_kept
    EXPECT(tg_keybias_attn_prefill(F, F, F, 512, 256, (const float*)F, (const float*)F, -1.0f, FI, FI, 1, 10, 10, 4,
                                   2, 128, 1e6, (void*)F, FF, (void*)F, 1 << 20, nullptr) == TG_ERR_INVALID_ARG);
    EXPECT(tg_attn_forward(F, 512, (const float*)F, 0.9f, FI, 1, 10, 10, 4, 2, 96, 1e6, (void*)F, FF, F, 1 << 20,
                           nullptr) == TG_ERR_UNSUPPORTED);                                      // head_dim
    EXPECT(tg_attn_decode(F, 512, FI, (const float*)F, 0.9f, FI, FI, 1, 10, 10, 6, 4, 128, 1e6, F, 1 << 20, (void*)F,
                          FF, (void*)F, 1 << 20, nullptr) == TG_ERR_INVALID_ARG);                // 6 % 4
    EXPECT(tg_attn_gate_grads(F, 512, F, 256, (const float*)F, (const float*)F, 0.0f, FI, 1, 10, 10, 4, 2, 128,
                              1e6, F, (const float*)F, F, 512, F, 1 << 20, FF, FF, FF, (void*)F, 1 << 20,
                              nullptr) == TG_ERR_INVALID_ARG);                                   // tau
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("host entry points clean under ASan/UBSan\n");
    return 0;
}
