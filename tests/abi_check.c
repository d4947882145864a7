/*
 * Argument validation of every libsdpa_bwd entry point, driven through the C
 * ABI from C.  tests/test_host_sanitize.py builds the library's host code with
 * AddressSanitizer and UndefinedBehaviorSanitizer and runs this program on a
 * host without a GPU: every call either fails validation with its documented
 * status before touching a pointer, or passes validation and stops at the
 * device check with SDPA_ERR_HIP.  Pointers are fake aligned addresses that
 * are never dereferenced.  Exit status 0 when every expectation holds.
 */
#include <stdint.h>
#include <stdio.h>

#include "../include/sdpa_bwd.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        int got_ = (call);                                                              \
        if (got_ != (want)) {                                                           \
            fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, \
                    (int)(want));                                                       \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

#define FAKE ((void*)0x10000)

static sdpa_tensor4 t4(int64_t sb, int64_t sh, int64_t ss) {
    sdpa_tensor4 t = {FAKE, sb, sh, ss, 1};
    return t;
}
static sdpa_tensor3 t3(int64_t st, int64_t sn) {
    sdpa_tensor3 t = {FAKE, st, sn, 1};
    return t;
}

static int dense2(int dtype, int64_t B, int64_t H, int64_t S, int64_t D, int64_t Dv, int det, size_t ws,
                  int noalloc) {
    sdpa_tensor4 a = t4(S * H * D, D, H * D);
    sdpa_stats st = {SDPA_STATS_LSE, (const float*)FAKE, NULL, H * S, S, 1};
    if (noalloc)
        return sdpa_bwd_noalloc(dtype, B, H, H, S, S, D, Dv, 0.125, 1, det, dtype, &a, &a, &a, &a, &a, &st, &a,
                                &a, &a, NULL);
    return sdpa_bwd(dtype, B, H, H, S, S, D, Dv, 0.125, 1, det, dtype, &a, &a, &a, &a, &a, &st, &a, &a, &a, FAKE,
                    ws, NULL);
}

static int dense(int dtype, int64_t B, int64_t H, int64_t S, int64_t D, int det, size_t ws, int noalloc) {
    return dense2(dtype, B, H, S, D, D, det, ws, noalloc);
}

static int varlen2(int64_t n, const int64_t* cu, int64_t H, int64_t D, int64_t Dv, int det, size_t ws) {
    sdpa_tensor3 a = t3(H * D, D);
    sdpa_stats st = {SDPA_STATS_MAX_SUM, (const float*)FAKE, (const float*)FAKE, 0, 1, H};
    return sdpa_bwd_varlen(SDPA_BF16, n, cu, cu, H, H, D, Dv, 0.088, 1, det, SDPA_BF16, &a, &a, &a, &a, &a, &st, &a,
                           &a, &a, FAKE, ws, NULL);
}

static int varlen(int64_t n, const int64_t* cu, int64_t H, int64_t D, int det, size_t ws) {
    return varlen2(n, cu, H, D, D, det, ws);
}

static int selected(int64_t n, const int64_t* cu, int64_t bs, int64_t count, const void* mask, int64_t ms,
                    size_t ws) {
    sdpa_tensor3 a = t3(16 * 128, 128), kv = t3(128, 128);
    sdpa_stats st = {SDPA_STATS_MAX_SUM, (const float*)FAKE, (const float*)FAKE, 0, 1, 16};
    return sdpa_bwd_selected(SDPA_BF16, n, cu, cu, 16, 1, 128, 128, 0.088, 2, (const uint8_t*)mask, ms,
                             (const int32_t*)FAKE, count, count, 1, bs, count, 0, SDPA_BF16, &a, &kv, &kv, &a, &a,
                             &st, &a, &kv, &kv, FAKE, ws, NULL);
}

int main(void) {
    size_t n = 0;
    /* dense */
    EXPECT(sdpa_bwd_workspace_size(SDPA_F16, 4, 12, 12, 1024, 1024, 64, 64, 0, &n), SDPA_OK);
    EXPECT(dense(SDPA_F16, 4, 12, 1024, 64, 0, n, 0), SDPA_ERR_HIP);
    EXPECT(dense(SDPA_F16, 4, 12, 1024, 64, 0, n - 1, 0), SDPA_ERR_WORKSPACE);
    EXPECT(dense(7, 4, 12, 1024, 64, 0, n, 0), SDPA_ERR_INVALID);
    EXPECT(dense(SDPA_F16, 4, 12, 1024, 96, 0, n, 0), SDPA_ERR_UNSUPPORTED);
    EXPECT(dense2(SDPA_F16, 4, 12, 1024, 192, 128, 0, n, 0), SDPA_ERR_HIP);          /* Dqk 192, Dv 128 */
    EXPECT(dense2(SDPA_F16, 4, 12, 1024, 128, 64, 0, n, 0), SDPA_ERR_UNSUPPORTED);
    EXPECT(dense2(SDPA_F16, 4, 12, 1024, 192, 128, 2, n, 0), SDPA_ERR_UNSUPPORTED);   /* no atomic dQ */
    EXPECT(dense2(SDPA_F16, 4, 12, 1024, 64, 0, 0, n, 0), SDPA_ERR_INVALID);
    EXPECT(dense(SDPA_F16, -1, 12, 1024, 64, 0, n, 0), SDPA_ERR_INVALID);
    EXPECT(dense(SDPA_F16, 4, 12, 1024, 64, 3, n, 0), SDPA_ERR_INVALID);
    EXPECT(dense(SDPA_F16, 4, 12, (int64_t)1 << 40, 64, 0, n, 0), SDPA_ERR_UNSUPPORTED);   /* huge S */
    EXPECT(sdpa_bwd_workspace_size(SDPA_F16, 4, 12, 12, 1024, 1024, 64, 64, 2, &n), SDPA_OK);
    EXPECT(dense(SDPA_F16, 4, 12, 1024, 64, 2, n, 0), SDPA_ERR_HIP);
    EXPECT(sdpa_bwd_workspace_size(SDPA_F16, 4, 12, 12, 1024, 1024, 64, 64, 0, NULL), SDPA_ERR_NULLPTR);
    /* allocation-free variant: fixed scratch */
    EXPECT(dense(SDPA_F16, 4, 12, 1024, 64, 0, 0, 1), SDPA_ERR_HIP);
    EXPECT(dense(SDPA_F16, 64, 64, 1024, 64, 0, 0, 1), SDPA_ERR_WORKSPACE);
    /* packed */
    {
        const int64_t cu[3] = {300, 700, 1500};
        const int64_t bad[3] = {300, 200, 1500};
        EXPECT(sdpa_bwd_varlen_workspace_size(SDPA_BF16, 3, cu, cu, 32, 32, 128, 128, 0, &n), SDPA_OK);
        EXPECT(varlen(3, cu, 32, 128, 0, n), SDPA_ERR_HIP);
        EXPECT(varlen(3, bad, 32, 128, 0, n), SDPA_ERR_INVALID);
        EXPECT(varlen(3, cu, 32, 96, 0, n), SDPA_ERR_UNSUPPORTED);
        EXPECT(varlen(3, cu, 32, 192, 2, n), SDPA_ERR_UNSUPPORTED);   /* no atomic dQ at D=192 */
        EXPECT(varlen2(3, cu, 32, 192, 128, 0, (size_t)1 << 40), SDPA_ERR_HIP);
        EXPECT(varlen2(3, cu, 32, 64, 128, 0, (size_t)1 << 40), SDPA_ERR_UNSUPPORTED);
        EXPECT(varlen(3, cu, 32, 128, 0, 8), SDPA_ERR_WORKSPACE);
        EXPECT(varlen(3, cu, 40000, 128, 0, (size_t)1 << 40), SDPA_ERR_UNSUPPORTED);
        EXPECT(varlen(0, cu, 32, 128, 0, n), SDPA_ERR_INVALID);
    }
    /* selected: 70 sequences, a user mask, bad block sizes */
    {
        int64_t cu[70];
        for (int i = 0; i < 70; ++i) cu[i] = 256 * (i + 1);
        EXPECT(sdpa_bwd_selected_workspace_size(SDPA_BF16, 70, cu, cu, 16, 1, 128, 128, 64, 4, 0, &n), SDPA_OK);
        EXPECT(selected(70, cu, 64, 4, NULL, 0, n), SDPA_ERR_HIP);
        EXPECT(selected(70, cu, 64, 4, FAKE, 256, n), SDPA_ERR_HIP);
        EXPECT(selected(70, cu, 64, 4, FAKE, 128, n), SDPA_ERR_INVALID);
        EXPECT(selected(70, cu, 64, 4, FAKE, 264, n), SDPA_ERR_UNSUPPORTED);
        EXPECT(selected(70, cu, 40, 4, NULL, 0, n), SDPA_ERR_INVALID);
        EXPECT(selected(70, cu, 64, 129, NULL, 0, n), SDPA_ERR_INVALID);
        EXPECT(selected(70, cu, 64, 4, NULL, 0, 16), SDPA_ERR_WORKSPACE);
        {
            int32_t off[1], ent[1];
            EXPECT(sdpa_selected_build_index(70, cu, cu, 1, (const int32_t*)FAKE, 4, 4, 1, 64, 4, off, ent, FAKE, n,
                                             NULL),
                   SDPA_ERR_HIP);
        }
    }
    /* forward */
    {
        sdpa_tensor4 a = t4(1024 * 12 * 64, 64, 12 * 64);
        sdpa_stats_out so = {(float*)FAKE, 12 * 1024, 1024, 1};
        EXPECT(sdpa_fwd_stats(SDPA_F16, 4, 12, 12, 1024, 1024, 64, 64, 0.125, 1, &a, &a, &a, &a, &so, NULL),
               SDPA_ERR_HIP);
        EXPECT(sdpa_fwd_stats(SDPA_F16, 4, 12, 5, 1024, 1024, 64, 64, 0.125, 1, &a, &a, &a, &a, &so, NULL),
               SDPA_ERR_INVALID);
    }
    for (int s = 0; s < 6; ++s)
        if (!sdpa_status_string(s)) ++failures;
    printf("abi_check: %d failure(s)\n", failures);
    return failures ? 1 : 0;
}
