/* Drives the argument validation of the C ABI (moe.h, moe_probe.h) without a GPU: every call
 * here must be rejected, or accepted as a no-op, before any HIP call.  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host side; exit status 0 when every
 * status code is the documented one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"
#include "moe_probe.h"

static int g_bad = 0;
#define EXPECT(call, want)                                                            \
    do {                                                                              \
        moe_status got_ = (call);                                                     \
        if (got_ != (want)) {                                                         \
            printf("line %d: %s -> %d, want %d\n", __LINE__, #call, (int)got_, (int)(want)); \
            g_bad = 1;                                                                \
        }                                                                             \
    } while (0)

static moe_problem prob(int T, int H, int E, int k, int F, moe_dtype act, moe_dtype wdt) {
    moe_problem p;
    memset(&p, 0, sizeof p);
    p.num_tokens = T;
    p.hidden = H;
    p.num_experts = E;
    p.top_k = k;
    p.ffn = F;
    p.act_dtype = act;
    p.w_dtype = wdt;
    p.renormalize = 1;
    p.path = MOE_PATH_AUTO;
    return p;
}

int main(void) {
    void* const FAKE = (void*)(uintptr_t)(1u << 20);  /* aligned, never dereferenced */
    void* const MIS = (void*)((uintptr_t)(1u << 20) + 2);
    size_t n = 0, a = 0, b = 0;
    moe_problem ok = prob(16, 256, 8, 2, 128, MOE_BF16, MOE_BF16);

    EXPECT(moe_workspace_size(&ok, &n), MOE_OK);
    EXPECT(moe_workspace_size(&ok, NULL), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_workspace_size(NULL, &n), MOE_ERR_INVALID_ARGUMENT);
    moe_problem p = prob(-1, 256, 8, 2, 128, MOE_BF16, MOE_BF16);
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_INVALID_ARGUMENT);
    p = prob(16, 256, 8, 9, 128, MOE_BF16, MOE_BF16);
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_INVALID_ARGUMENT);
    p = prob(16, 256, 513, 2, 128, MOE_BF16, MOE_BF16);
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_INVALID_ARGUMENT);
    p = prob(16, 192, 8, 2, 128, MOE_BF16, MOE_BF16);
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_UNSUPPORTED);
    p = prob(16, 256, 8, 2, 128, MOE_F32, MOE_NVFP4);
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_UNSUPPORTED);

    EXPECT(moe_packed_weights_size(&ok, &a, &b), MOE_OK);
    if (a != (size_t)8 * 2 * 128 * 256 * 2 || b != (size_t)8 * 256 * 128 * 2) g_bad = 1;

    /* held expert ranges (expert parallelism) */
    p = ok; p.expert_begin = 2;                      /* a start without a count */
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_INVALID_ARGUMENT);
    p = ok; p.expert_begin = 4; p.local_experts = 5; /* past E */
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_INVALID_ARGUMENT);
    p = ok; p.expert_begin = -1; p.local_experts = 2;
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_INVALID_ARGUMENT);
    p = ok; p.local_experts = -1;
    EXPECT(moe_workspace_size(&p, &n), MOE_ERR_INVALID_ARGUMENT);
    p = ok; p.expert_begin = 4; p.local_experts = 4;
    EXPECT(moe_workspace_size(&p, &n), MOE_OK);
    EXPECT(moe_packed_weights_size(&p, &a, &b), MOE_OK); /* the 4 held experts only */
    if (a != (size_t)4 * 2 * 128 * 256 * 2 || b != (size_t)4 * 256 * 128 * 2) g_bad = 1;
    EXPECT(moe_pack_weights(&ok, FAKE, NULL, FAKE, NULL, NULL), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_pack_weights(&ok, MIS, NULL, FAKE, NULL, NULL), MOE_ERR_INVALID_ARGUMENT);

    EXPECT(moe_route(&ok, NULL, FAKE, NULL, FAKE, FAKE, FAKE, n, NULL), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_route(&ok, MIS, FAKE, NULL, FAKE, FAKE, FAKE, n, NULL), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_route(&ok, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 16, NULL), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_permute(&ok, FAKE, FAKE, NULL, FAKE, FAKE, NULL, NULL, FAKE, n, NULL),
           MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_permute(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, n, NULL),
           MOE_ERR_INVALID_ARGUMENT);

    moe_expert_weights w;
    memset(&w, 0, sizeof w);
    w.w13 = FAKE;
    w.w2 = FAKE;
    w.layout = 2;  /* no such layout */
    EXPECT(moe_forward(&ok, FAKE, FAKE, NULL, &w, FAKE, NULL, NULL, NULL, NULL, NULL, NULL, FAKE,
                       n, NULL),
           MOE_ERR_INVALID_ARGUMENT);
    w.layout = MOE_LAYOUT_ROW_MAJOR;  /* bf16 weights row-major: accepted */
    EXPECT(moe_forward(&ok, FAKE, FAKE, NULL, &w, FAKE, NULL, NULL, NULL, NULL, NULL, NULL, FAKE,
                       16, NULL),
           MOE_ERR_WORKSPACE_TOO_SMALL);
    w.layout = MOE_LAYOUT_PACKED;
    EXPECT(moe_forward(&ok, FAKE, FAKE, NULL, &w, FAKE, NULL, NULL, NULL, NULL, NULL, NULL, FAKE,
                       16, NULL),
           MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_grouped_gemm(&ok, (moe_gemm_kind)7, FAKE, NULL, FAKE, &w, FAKE, FAKE, n, NULL),
           MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_combine(&ok, NULL, FAKE, FAKE, FAKE, NULL), MOE_ERR_INVALID_ARGUMENT);
    moe_problem nv = prob(16, 256, 8, 2, 128, MOE_BF16, MOE_NVFP4);
    w.layout = MOE_LAYOUT_ROW_MAJOR;
    EXPECT(moe_forward(&nv, FAKE, FAKE, NULL, &w, FAKE, NULL, NULL, NULL, NULL, NULL, NULL, FAKE,
                       (size_t)1 << 40, NULL),
           MOE_ERR_INVALID_ARGUMENT); /* NVFP4 without scales */

    /* T = 0: a successful no-op with empty buffers (no counts/offsets given: no device work) */
    moe_problem z = prob(0, 256, 8, 2, 128, MOE_BF16, MOE_BF16);
    EXPECT(moe_forward(&z, NULL, NULL, NULL, &w, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                       NULL),
           MOE_OK);
    EXPECT(moe_route(&z, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);

    EXPECT(moe_probe_mfma_bf16(0, 1, (float*)FAKE, NULL), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_probe_read(FAKE, 100, (uint32_t*)FAKE, NULL), MOE_ERR_INVALID_ARGUMENT);

    for (int s = 0; s <= 5; ++s)
        if (!moe_status_string((moe_status)s) || !moe_status_string((moe_status)s)[0]) g_bad = 1;
    printf("abi validation: %s\n", g_bad ? "FAILED" : "ok");
    return g_bad;
}
