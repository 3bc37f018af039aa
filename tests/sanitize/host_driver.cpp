// host_driver.cpp -- exercises the host side of libda2 (da2_host.cpp and
// da2_partition.cpp) under AddressSanitizer / UndefinedBehaviorSanitizer,
// for the build tests/test_sanitizers.py makes: layouts of every frame up
// to 48 x 48 (grid and ragged partitions, with and without a text prefix),
// workspace carving, slot tables, debug sizes, plan objects over a fake
// workspace address, and every argument check that returns before a launch.
// No GPU work: the kernel launchers are stubs that abort if reached.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "da2.h"
#include "da2_internal.h"

namespace da2 {
#define DA2_STUB(...)                                      \
    {                                                      \
        fprintf(stderr, "a kernel launcher was reached\n"); \
        abort();                                           \
    }
void launch_prep_qk(const da2_layout_s &, const void *, int, char *, hipStream_t) DA2_STUB()
void launch_prep_v(const da2_layout_s &, const void *, int, int, char *, hipStream_t) DA2_STUB()
void launch_prep_vp(const da2_layout_s &, const PrefixIo &, char *, hipStream_t) DA2_STUB()
void launch_draft(const da2_layout_s &, double, char *, hipStream_t) DA2_STUB()
void launch_draft_logits(const da2_layout_s &, char *, hipStream_t) DA2_STUB()
void launch_skip_means(const da2_layout_s &, char *, hipStream_t) DA2_STUB()
void launch_rank(const da2_layout_s &, int, int64_t, int64_t, int64_t, char *, hipStream_t) DA2_STUB()
void launch_schedule(const da2_layout_s &, char *, hipStream_t) DA2_STUB()
void launch_attention(const da2_layout_s &, char *, const void *, const void *, void *, int, const PrefixIo *,
                      int, hipEvent_t *, hipStream_t) DA2_STUB()
void launch_debug(const da2_layout_s &, int, const char *, void *, hipStream_t) DA2_STUB()
void launch_import_tier(const da2_layout_s &, const uint8_t *, char *, hipStream_t) DA2_STUB()
}  // namespace da2

#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);  \
            exit(2);                                                        \
        }                                                                   \
    } while (0)

static void one_layout(int B, int H, int d, int F, int Hv, int Wv, int prefix, int cap = 0)
{
    const int64_t N = (int64_t)F * Hv * Wv;
    const int C = cap ? cap : 64;
    da2_shape s = {B, H, d, F, Hv, Wv, H * N * d, N * d, d, prefix, cap};
    da2_layout_t *L = nullptr;
    const da2_status st = da2_layout_create(&s, &L);
    if (st != DA2_OK) {
        CHECK(st == DA2_ERR_UNSUPPORTED_SHAPE && !L);
        return;
    }
    int32_t rf = 0;
    const int32_t R = da2_layout_regions(L, &rf);
    CHECK(R == F * rf && rf == (Hv * Wv + C - 1) / C);
    int32_t *slots = (int32_t *)malloc(sizeof(int32_t) * rf * C);
    CHECK(da2_layout_slots(L, slots) == DA2_OK);
    // every token of the frame exactly once
    int32_t *seen = (int32_t *)calloc((size_t)Hv * Wv, sizeof(int32_t));
    for (int i = 0; i < rf * C; i++)
        if (slots[i] >= 0) {
            CHECK(slots[i] < Hv * Wv);
            seen[slots[i]]++;
        }
    for (int t = 0; t < Hv * Wv; t++)
        CHECK(seen[t] == 1);
    const size_t ws = da2_workspace_bytes(L);
    CHECK(ws > 0);
    for (int w = 0; w < DA2_DBG_COUNT; w++)
        (void)da2_plan_debug_bytes(L, w);
    CHECK(da2_plan_debug_bytes(L, -1) == 0 && da2_plan_debug_bytes(L, DA2_DBG_COUNT) == 0);
    // a plan over a fake (never touched) 256-aligned workspace address
    void *fake = (void *)(uintptr_t)(1ull << 40);
    da2_plan_t *P = nullptr;
    CHECK(da2_plan_create(L, fake, ws - 1, &P) == DA2_ERR_WORKSPACE);
    CHECK(da2_plan_create(L, (char *)fake + 16, ws, &P) == DA2_ERR_WORKSPACE);
    CHECK(da2_plan_create(L, fake, ws, &P) == DA2_OK && P);
    const void *q = (const void *)(uintptr_t)(1ull << 41), *k = (const void *)(uintptr_t)(1ull << 42);
    da2_budget bad[5] = {{-1, 0, 0.2, 0, 0, 0}, {6000, 6000, 0.2, 0, 0, 0}, {1000, 0, 1.5, 0, 0, 0},
                         {1000, 0, NAN, 0, 0, 0}, {1000, 0, 0.2, 3, 0, 0}};
    for (auto &b : bad)
        CHECK(da2_plan(P, q, k, &b, nullptr) == DA2_ERR_INVALID_ARG);
    da2_budget good = {1000, 3000, 0.2, 0, 0, 0};
    if (C > 64) {   // block-mean tiles need capacity 64
        da2_budget means = {1000, 3000, 0.2, 0, 0, 1};
        CHECK(da2_plan(P, q, k, &means, nullptr) == DA2_ERR_INVALID_ARG);
    }
    CHECK(da2_plan(P, (const char *)q + 2, k, &good, nullptr) == DA2_ERR_INVALID_ARG);   // misaligned
    CHECK(da2_plan(P, nullptr, k, &good, nullptr) == DA2_ERR_INVALID_ARG);
    // no plan yet: attention refuses before any launch
    CHECK(da2_attention(P, q, k, q, (void *)k, 1, nullptr) == DA2_ERR_PLAN_MISMATCH);
    CHECK(da2_attention(P, q, k, q, (void *)k, 7, nullptr) == DA2_ERR_INVALID_ARG);
    CHECK(da2_plan_tier_map(P, (uint8_t *)(uintptr_t)(1ull << 43), nullptr) == DA2_ERR_PLAN_MISMATCH);
    if (prefix)
        CHECK(da2_attention_prefixed(P, q, k, q, (void *)k, nullptr, k, q, (void *)k, nullptr, 1, nullptr) ==
              DA2_ERR_INVALID_ARG);
    // the no-alloc entry point refuses a workspace beyond its array first
    if (ws > DA2_NOALLOC_BYTES)
        CHECK(da2_forward_noalloc(L, q, k, q, (void *)k, &good, 1, nullptr) == DA2_ERR_WORKSPACE);
    da2_plan_destroy(P);
    da2_layout_destroy(L);
    free(slots);
    free(seen);
}

int main()
{
    for (int Hv = 1; Hv <= 48; Hv++)
        for (int Wv = 1; Wv <= 48; Wv++)
            one_layout(1, 2, (Hv + Wv) % 2 ? 64 : 128, 2, Hv, Wv, (Hv * Wv) % 3 ? 0 : 90);
    for (int Hv = 8; Hv <= 40; Hv += 3)
        for (int Wv = 8; Wv <= 40; Wv += 5)
            one_layout(1, 2, 64, 2, Hv, Wv, (Hv * Wv) % 2 ? 0 : 70, 128);
    one_layout(1, 40, 128, 21, 48, 80, 0);     // a Wan-14B 720p layer
    one_layout(1, 40, 128, 21, 48, 80, 0, 128);   // the same at capacity 128
    one_layout(1, 24, 128, 33, 34, 60, 256);   // HunyuanVideo 544p with a prefix
    int64_t t16, t8, tk;
    da2_quotas(1260 * 1260, 500, 1000, 3000, &t16, &t8, &tk);
    CHECK(t16 <= t8 && t8 <= tk);
    double c[17];
    da2_exp_constants(c);
    for (int s = 0; s <= 5; s++)
        CHECK(da2_status_string((da2_status)s) != nullptr);
    CHECK(da2_layout_create(nullptr, nullptr) == DA2_ERR_INVALID_ARG);
    printf("host driver ok\n");
    return 0;
}
