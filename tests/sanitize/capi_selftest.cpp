// Host-side argument validation of the C ABI (include/sparse_moe.h) under
// AddressSanitizer and UndefinedBehaviorSanitizer.  tests/test_sanitizers.py
// builds the library's sources for the host only (no GPU code) with both
// sanitizers and links this driver against them.  Every call below is
// rejected before anything is enqueued, so no HIP runtime call is made and
// the fake device addresses are never dereferenced; the workspace-size
// queries run their full arithmetic.  Exit status 0 = every check passed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sparse_moe.h"

static int failures = 0;
#define EXPECT(expr, want)                                                               \
    do {                                                                                 \
        const int got_ = (int)(expr);                                                    \
        if (got_ != (int)(want)) {                                                       \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, \
                    (int)(want));                                                        \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

int main() {
    void* A = (void*)0x100000;     // 16-byte aligned fake device addresses
    void* B = (void*)0x200000;
    void* MIS = (void*)0x100004;   // misaligned
    const float* F = (const float*)A;
    float* Fw = (float*)A;
    int32_t* I32 = (int32_t*)A;

    for (int s = 0; s <= 8; ++s) EXPECT(strlen(moe_status_string(s)) > 0, 1);
    EXPECT(moe_abi_version(), MOE_ABI_VERSION);

    // router / top-K
    EXPECT(moe_router_topk(A, 0, 4, 256, F, nullptr, nullptr, 0, 1, Fw, I32, Fw, nullptr), MOE_ERR_SHAPE);
    EXPECT(moe_router_topk(A, 0, 4, 256, F, nullptr, nullptr, 8, 9, Fw, I32, Fw, nullptr), MOE_ERR_SHAPE);
    EXPECT(moe_router_topk(A, 0, 4, 100, F, nullptr, nullptr, 8, 2, Fw, I32, Fw, nullptr), MOE_ERR_SHAPE);
    EXPECT(moe_router_topk(A, 5, 4, 256, F, nullptr, nullptr, 8, 2, Fw, I32, Fw, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_router_topk(nullptr, 0, 0, 256, nullptr, nullptr, nullptr, 8, 2, nullptr, nullptr, nullptr, nullptr), MOE_OK);
    EXPECT(moe_router_topk(nullptr, 0, 4, 256, F, nullptr, nullptr, 8, 2, Fw, I32, Fw, nullptr), MOE_ERR_NULL);
    EXPECT(moe_router_topk(A, 0, 4, 256, F, nullptr, nullptr, 8, 2, Fw, I32, (float*)MIS, nullptr), MOE_ERR_ALIGN);
    EXPECT(moe_router_topk(A, 0, (int64_t)1 << 40, 256, F, nullptr, nullptr, 8, 2, Fw, I32, Fw, nullptr), MOE_ERR_SHAPE);

    // permutation
    const size_t pws = moe_permute_workspace_bytes(4096, 8, 128);
    EXPECT(pws > 0, 1);
    EXPECT(moe_permute_workspace_bytes(4, 9, 8), 0);
    EXPECT(moe_permute(I32, 4096, 8, 128, I32, I32, I32, nullptr, 0, nullptr), MOE_ERR_WORKSPACE);
    EXPECT(moe_permute(I32, 4, 2, 8, I32, (int32_t*)MIS, I32, nullptr, 0, nullptr), MOE_ERR_ALIGN);
    EXPECT(moe_permute(nullptr, 4, 2, 8, I32, I32, I32, nullptr, 0, nullptr), MOE_ERR_NULL);

    // routing in one call
    const size_t rws = moe_route_workspace_bytes(8, 8, 128);
    EXPECT(rws >= 256, 1);
    EXPECT(moe_route(A, 0, 8, 2816, F, nullptr, nullptr, 128, 8, Fw, I32, Fw, I32, I32, I32, A, 16, nullptr), MOE_ERR_WORKSPACE);
    EXPECT(moe_route(A, 0, 8, 2816, F, nullptr, nullptr, 128, 17, Fw, I32, Fw, I32, I32, I32, A, rws, nullptr), MOE_ERR_SHAPE);

    // expert FFN, and its no-allocation variant (rejected before any device lookup)
    const size_t fws = moe_expert_ffn_q4_0_workspace_bytes(4096, 8, 2816, 704, 128, MOE_BF16);
    EXPECT(fws >= (size_t)4096 * 8 * 704 * 2, 1);
    EXPECT(moe_expert_ffn_q4_0_workspace_bytes(4, 2, 250, 64, 8, MOE_F32), 0);
    EXPECT(moe_expert_ffn_q4_0(A, 1, 4096, 2816, A, B, 704, 128, 8, I32, I32, Fw, A, 16, nullptr), MOE_ERR_WORKSPACE);
    EXPECT(moe_expert_ffn_q4_0(A, 1, 4, 2816, A, B, 700, 128, 8, I32, I32, Fw, A, fws, nullptr), MOE_ERR_SHAPE);
    EXPECT(moe_expert_ffn_q4_0(A, 1, 4, 2816, MIS, B, 704, 128, 8, I32, I32, Fw, A, fws, nullptr), MOE_ERR_ALIGN);
    EXPECT(moe_expert_ffn_q4_0_noalloc(A, 1, 4096, 2816, A, B, 704, 128, 8, I32, I32, Fw, nullptr), MOE_ERR_SCRATCH);
    EXPECT(moe_expert_ffn_q4_0_noalloc(nullptr, 1, 8, 2816, A, B, 704, 128, 8, I32, I32, Fw, nullptr), MOE_ERR_NULL);
    EXPECT(moe_expert_ffn_q4_0_noalloc(A, 4, 8, 2816, A, B, 704, 128, 8, I32, I32, Fw, nullptr), MOE_ERR_UNSUPPORTED);

    // one-call decode layer
    const size_t dws = moe_layer_decode_workspace_bytes(1, 8, 2816, 704, 128, MOE_F32);
    EXPECT(dws >= 8 * 704 * 4, 1);
    EXPECT(moe_layer_decode(A, 0, 9, 2816, F, nullptr, nullptr, 128, 8, A, B, 704, F, Fw, I32, Fw, I32, I32, I32, nullptr, 0, Fw, nullptr, 0, A, dws, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_layer_decode(A, 0, 1, 2848, F, nullptr, nullptr, 128, 8, A, B, 704, F, Fw, I32, Fw, I32, I32, I32, nullptr, 0, Fw, nullptr, 0, A, dws, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_layer_decode(A, 0, 1, 2816, F, nullptr, nullptr, 128, 8, A, B, 704, F, Fw, I32, Fw, I32, I32, I32, nullptr, 0, nullptr, nullptr, 0, A, dws, nullptr), MOE_ERR_NULL);
    EXPECT(moe_layer_decode(A, 0, 1, 2816, F, nullptr, nullptr, 128, 8, A, B, 704, F, Fw, I32, Fw, I32, I32, I32, nullptr, 0, Fw, nullptr, 0, A, 16, nullptr), MOE_ERR_WORKSPACE);
    EXPECT(moe_layer_decode(A, 0, 1, 2816, F, nullptr, nullptr, 128, 8, A, B, 704, F, Fw, I32, Fw, I32, I32, I32, nullptr, 0, (float*)MIS, nullptr, 0, A, dws, nullptr), MOE_ERR_ALIGN);

    // linear layer, combine, RMSNorm
    const size_t lws = moe_linear_q4_0_workspace_bytes(4096, 2816, 4224, MOE_BF16);
    EXPECT(lws > 0, 1);
    EXPECT(moe_linear_q4_0(A, 0, 4, 2816, A, 70000, Fw, A, lws, nullptr), MOE_ERR_SHAPE);
    EXPECT(moe_linear_q4_0(A, 0, 4, 2816, A, 4224, Fw, A, 16, nullptr), MOE_ERR_WORKSPACE);
    EXPECT(moe_combine(F, I32, I32, F, F, 4, 2, 256, nullptr, 0, nullptr, nullptr, 0, nullptr), MOE_ERR_NULL);
    EXPECT(moe_combine(F, I32, nullptr, F, F, 4, 2, 256, nullptr, 0, Fw, nullptr, 0, nullptr), MOE_ERR_NULL);
    EXPECT(moe_combine(F, I32, I32, F, F, 4, 2, 256, MIS, 0, Fw, nullptr, 0, nullptr), MOE_ERR_ALIGN);
    EXPECT(moe_rmsnorm(A, 1, F, 1e-6f, 4, 100, A, 1, nullptr), MOE_ERR_SHAPE);
    EXPECT(moe_rmsnorm(A, 1, F, -1.0f, 4, 256, A, 1, nullptr), MOE_ERR_SHAPE);
    EXPECT(moe_rmsnorm(A, 1, nullptr, 1e-6f, 4, 256, A, 1, nullptr), MOE_ERR_NULL);

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("C-ABI validation self-test passed\n");
    return 0;
}
