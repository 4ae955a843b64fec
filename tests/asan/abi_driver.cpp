// abi_driver.cpp -- drives every entry point of the C ABI layer through its
// argument checks, built with AddressSanitizer and UndefinedBehaviorSanitizer
// against recording stand-ins of the kernel launchers (launch_stubs.cpp).
// Pointers are fake addresses that nothing dereferences.  Exit status 0 when
// every expectation holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "osm.h"
#include "osm_internal.h"

namespace osm {
extern int g_launches;
extern SoftmaxPlan g_softmax_plan;
extern AttnFwdArgs g_fwd;
extern DecodeArgs g_decode;
extern DecodeLayout g_decode_layout;
extern MergeArgs g_merge;
extern MergeLseArgs g_merge_lse;
}  // namespace osm

static int failures = 0;

#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

int main() {
    float *F = static_cast<float *>(fake(0x100000));
    void *P = fake(0x200000);
    void *W = fake(0x300000);           // 256-byte aligned workspace
    const int32_t *LEN = static_cast<const int32_t *>(fake(0x400000));

    // ---- status strings ----------------------------------------------------
    for (int c = 0; c <= 5; ++c) EXPECT(osm_status_str(static_cast<osm_status>(c)) != nullptr);
    EXPECT(osm_status_str(static_cast<osm_status>(77)) != nullptr);

    // ---- softmax: both entry points -----------------------------------------
    typedef osm_status (*SoftmaxFn)(const float *, float *, int64_t, int64_t, int64_t, int64_t, float *,
                                    float *, osm_stream);
    const SoftmaxFn fns[2] = {osm_softmax_rows, osm_softmax_rows_twopass};
    for (int i = 0; i < 2; ++i) {
        SoftmaxFn f = fns[i];
        EXPECT(f(F, F, -1, 4, 4, 4, nullptr, nullptr, nullptr) == OSM_ERR_SHAPE);
        EXPECT(f(F, F, 2, 4, 3, 4, nullptr, nullptr, nullptr) == OSM_ERR_SHAPE);
        EXPECT(f(nullptr, F, 2, 4, 4, 4, nullptr, nullptr, nullptr) == OSM_ERR_NULL);
        EXPECT(f(nullptr, nullptr, 0, 4, 4, 4, nullptr, nullptr, nullptr) == OSM_OK);
        const int before = osm::g_launches;
        EXPECT(f(F, F, 4096, 32000, 32000, 32000, F, F, nullptr) == OSM_OK);
        EXPECT(osm::g_launches == before + 1);
        EXPECT(osm::g_softmax_plan.resident == (i == 0));
        EXPECT(f(F, F, 3, INT64_MAX / 8, INT64_MAX / 8, INT64_MAX / 8, nullptr, nullptr, nullptr) == OSM_OK);
        EXPECT(!osm::g_softmax_plan.resident && osm::g_softmax_plan.threads == 1024);
    }
    EXPECT(osm_softmax_rows_twopass(F, F, 1, 5, 5, 5, nullptr, nullptr, nullptr) == OSM_OK);
    EXPECT(osm::g_softmax_plan.threads == 64);

    // ---- attention forward ------------------------------------------------------
    EXPECT(osm_attn_fwd(P, P, P, P, F, OSM_BF16, 0, 2, 1, 8, 8, 128, nullptr, nullptr, 0.1f, 0, nullptr) == OSM_ERR_SHAPE);
    EXPECT(osm_attn_fwd(P, P, P, P, F, OSM_BF16, 1, 2, 1, 8, 8, 128, nullptr, nullptr, NAN, 0, nullptr) == OSM_ERR_SHAPE);
    EXPECT(osm_attn_fwd(P, P, P, P, F, OSM_BF16, 1, 2, 1, 8, 1 << 23, 128, nullptr, nullptr, 0.1f, 0, nullptr) == OSM_ERR_UNSUPPORTED);
    EXPECT(osm_attn_fwd(P, P, P, P, F, OSM_BF16, INT32_MAX, INT32_MAX, 1, 8, 8, 128, nullptr, nullptr, 0.1f, 0, nullptr) == OSM_ERR_UNSUPPORTED);
    EXPECT(osm_attn_fwd(P, P, P, P, F, OSM_BF16, 4, 32, 8, 4096, 4096, 128, LEN, LEN, 0.1f, 1, nullptr) == OSM_OK);
    EXPECT(osm::g_fwd.batch == 4 && osm::g_fwd.heads_kv == 8 && osm::g_fwd.causal == 1);
    EXPECT(osm_attn_fwd_fp8(P, P, P, P, F, 1, 2, 1, 8, 8, 128, nullptr, nullptr, 0.1f, INFINITY, 0, nullptr) == OSM_ERR_SHAPE);
    EXPECT(osm_attn_fwd_fp8(P, P, P, P, F, 1, 2, 1, 8, 1 << 24, 128, nullptr, nullptr, 0.1f, 1.0f, 0, nullptr) == OSM_ERR_UNSUPPORTED);
    EXPECT(osm_attn_fwd_fp8(P, P, P, P, F, 1, 2, 1, 8, 8, 128, nullptr, nullptr, 0.1f, 1.0f, 0, nullptr) == OSM_OK);

    // ---- backward ----------------------------------------------------------------
    EXPECT(osm_attn_bwd_workspace_bytes(INT32_MAX, INT32_MAX, INT32_MAX) == 0);
    EXPECT(osm_attn_bwd_workspace_bytes(4, 32, 4096) == (size_t)4 * 32 * 4096 * 8);
    const size_t bws = osm_attn_bwd_workspace_bytes(1, 2, 8);
    EXPECT(osm_attn_bwd(P, P, P, P, P, F, P, P, P, OSM_BF16, 1, 2, 1, 8, 8, 128, nullptr, nullptr, 0.1f, 0,
                        W, bws - 1, nullptr) == OSM_ERR_WORKSPACE);
    EXPECT(osm_attn_bwd(P, P, P, P, P, F, P, P, P, OSM_BF16, 1, 2, 1, 8, 8, 128, nullptr, nullptr, 0.1f, 0,
                        W, bws, nullptr) == OSM_OK);

    // ---- decode: workspace layout, merge pointers inside the workspace ------------
    EXPECT(osm_decode_workspace_bytes(1 << 15, 1 << 15, INT32_MAX, 128, 64) == 0);   // past 2^62 bytes
    EXPECT(osm_attn_decode_splitkv(P, P, P, P, F, OSM_BF16, 1 << 15, 1 << 15, 1 << 13, INT32_MAX, 128, LEN,
                                   0.1f, 64, W, SIZE_MAX, nullptr) == OSM_ERR_UNSUPPORTED);
    const size_t dws = osm_decode_workspace_bytes(16, 32, 32768, 128, 256);
    EXPECT(dws == 2 * (size_t)(16 * 32 * 128 * 4) + (size_t)16 * 32 * 128 * 128 * 4);
    EXPECT(osm_attn_decode_splitkv(P, P, P, P, F, OSM_BF16, 16, 32, 8, 32768, 128, LEN, 0.1f, 256, W, dws - 1,
                                   nullptr) == OSM_ERR_WORKSPACE);
    EXPECT(osm_attn_decode_splitkv(P, P, P, P, F, OSM_BF16, 16, 32, 8, 32768, 128, LEN, 0.1f, 256,
                                   fake(0x300010), dws, nullptr) == OSM_ERR_WORKSPACE);
    const int before = osm::g_launches;
    EXPECT(osm_attn_decode_splitkv(P, P, P, P, F, OSM_BF16, 16, 32, 8, 32768, 128, LEN, 0.1f, 256, W, dws,
                                   nullptr) == OSM_OK);
    EXPECT(osm::g_launches == before + 2);
    EXPECT(osm::g_decode_layout.chunks == 128 && osm::g_decode_layout.rows == 512);
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(W);
    const uintptr_t pm = reinterpret_cast<uintptr_t>(osm::g_merge.part_m);
    const uintptr_t pl = reinterpret_cast<uintptr_t>(osm::g_merge.part_l);
    const uintptr_t po = reinterpret_cast<uintptr_t>(osm::g_merge.part_o);
    EXPECT(pm == w0 && pl >= pm + 512 * 128 * 4 && po >= pl + 512 * 128 * 4);
    EXPECT(po + (size_t)512 * 128 * 128 * 4 <= w0 + dws);
    EXPECT(osm::g_merge.num_splits == 128 && osm::g_merge.head_dim == 128);

    // ---- decode without a workspace: the library's scratch -----------------------
    EXPECT(osm_attn_decode_splitkv_noalloc(P, P, P, P, F, OSM_BF16, 16, 32, 8, 32768, 128, LEN, 0.1f, 256,
                                           nullptr) == OSM_OK);
    EXPECT(reinterpret_cast<uintptr_t>(osm::g_merge.part_m) == 0x7000000);
    EXPECT(reinterpret_cast<uintptr_t>(osm::g_merge.part_o) + (size_t)512 * 128 * 128 * 4 <=
           0x7000000 + OSM_DECODE_SCRATCH_BYTES);
    // 4 x the workspace above (136 MiB) does not fit the 64 MiB scratch
    EXPECT(osm_attn_decode_splitkv_noalloc(P, P, P, P, F, OSM_BF16, 64, 32, 8, 32768, 128, LEN, 0.1f, 256,
                                           nullptr) == OSM_ERR_WORKSPACE);
    EXPECT(osm_attn_decode_splitkv_noalloc(P, P, P, P, F, OSM_BF16, 16, 32, 8, 32768, 128, nullptr, 0.1f, 256,
                                           nullptr) == OSM_ERR_NULL);
    EXPECT(osm_attn_decode_splitkv_noalloc(P, P, P, P, F, OSM_BF16, 16, 32, 8, 32768, 128, LEN, 0.1f, 100,
                                           nullptr) == OSM_ERR_UNSUPPORTED);

    // ---- extend ------------------------------------------------------------------
    const size_t ews = osm_decode_workspace_bytes(16, 32, 4096, 128, 512);
    EXPECT(osm_attn_extend(P, P, P, OSM_BF16, 16, 32, 8, 4096, 128, 0.1f, F, F, F, 512, W, ews, nullptr) == OSM_OK);
    EXPECT(osm::g_merge.state_m == F && osm::g_merge.o == nullptr);
    EXPECT(osm_attn_extend(nullptr, nullptr, nullptr, OSM_BF16, 16, 32, 8, 0, 128, 0.1f, F, F, F, 512, nullptr, 0,
                           nullptr) == OSM_OK);

    // ---- merges ---------------------------------------------------------------------
    EXPECT(osm_merge_partials(F, F, F, 4, 3, 513, P, OSM_F32, F, nullptr) == OSM_ERR_UNSUPPORTED);
    EXPECT(osm_merge_partials(F, F, F, 4, 3, 64, P, OSM_F32, F, nullptr) == OSM_OK);
    EXPECT(osm_merge_lse(fake(0x200008), F, 4, 3, 128, OSM_BF16, P, OSM_BF16, F, nullptr) == OSM_ERR_UNSUPPORTED);
    EXPECT(osm_merge_lse(P, F, 4, 3, 128, OSM_BF16, fake(0x200004), OSM_BF16, F, nullptr) == OSM_ERR_UNSUPPORTED);
    EXPECT(osm_merge_lse(P, F, 4, 3, 128, OSM_BF16, P, OSM_F32, F, nullptr) == OSM_OK);
    EXPECT(osm::g_merge_lse.in_bf16 == 1 && osm::g_merge_lse.out_bf16 == 0);

    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("abi driver: all expectations hold\n");
    return 0;
}
