/* Drives the host side of libsvla (built for the host only, with
 * AddressSanitizer and UndefinedBehaviorSanitizer) through every path that
 * runs before a HIP call: version and status strings, workspace sizes and
 * launch plans over many shapes, and the argument checks of every entry
 * point.  Any invalid access or undefined operation aborts the process.
 * Addresses passed as device pointers are never dereferenced by these paths. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "svla.h"

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { ++fails; printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, svla_last_error()); } } while (0)

int main(void)
{
    void *A = (void *)(uintptr_t)0x10000, *B2 = (void *)(uintptr_t)0x40000000;
    void *MIS = (void *)(uintptr_t)0x10004;
    float *F = (float *)A;
    EXPECT(svla_abi_version() == SVLA_ABI_VERSION);
    for (int s = -1; s <= 9; ++s) EXPECT(svla_status_string((svla_status)s) != NULL);
    EXPECT(svla_last_error() != NULL);

    /* workspace sizes and launch plans over a grid of shapes */
    const int ds[] = {16, 32, 64, 128};
    const int ns[] = {0, 1, 15, 16, 17, 390, 1170, 2048, 2049, 8190};
    const int nbs[] = {0, 1, 2, 7, 17, 80};
    const int bhs[][2] = {{0, 4}, {1, 1}, {1, 70}, {2, 70}, {1, 20}, {64, 64}};
    svla_rope ropes[] = {{8, 12, 12, 15, 26, 0, 10000.f}, {16, 24, 24, 22, 40, 79, 500.f},
                         {2, 0, 0, 1, 1, 0, 10.f}};
    char buf[4096];
    for (int op = SVLA_OP_NONCAUSAL - 1; op <= SVLA_OP_BACKWARD + 1; ++op)
        for (int dt = SVLA_F32; dt <= SVLA_FP8 + 1; ++dt)
            for (unsigned di = 0; di < sizeof ds / sizeof *ds; ++di)
                for (unsigned ni = 0; ni < sizeof ns / sizeof *ns; ++ni)
                    for (unsigned bi = 0; bi < sizeof nbs / sizeof *nbs; ++bi)
                        for (unsigned hi = 0; hi < sizeof bhs / sizeof *bhs; ++hi) {
                            size_t bytes = 0;
                            svla_workspace_size((svla_op)op, (svla_dtype)dt, bhs[hi][0], bhs[hi][1],
                                                nbs[bi], ns[ni], ds[di], &bytes);
                            for (int r = -1; r < 3; ++r) {
                                const svla_rope *rp = r < 0 ? NULL : &ropes[r];
                                buf[0] = 0;
                                if (svla_describe((svla_op)op, (svla_dtype)dt, bhs[hi][0], bhs[hi][1],
                                                  nbs[bi], ns[ni], ds[di], rp, buf, sizeof buf) == SVLA_OK)
                                    EXPECT(memchr(buf, 0, sizeof buf) != NULL && buf[0] == '{');
                            }
                        }
    EXPECT(svla_describe(SVLA_OP_BLOCK_STEP, SVLA_BF16, 1, 70, 1, 1170, 32, NULL, buf, 8) == SVLA_ERR_VALUE);
    EXPECT(svla_describe(SVLA_OP_BLOCK_STEP, SVLA_BF16, 1, 70, 1, 1170, 32, NULL, NULL, 8) == SVLA_ERR_NULL);
    EXPECT(svla_workspace_size(SVLA_OP_APPLY, SVLA_BF16, 1, 1, 1, 1, 32, NULL) == SVLA_ERR_NULL);

    /* argument checks of every entry point (none reaches a HIP call) */
    EXPECT(svla_noncausal(SVLA_BF16, 1, 2, 64, 32, NULL, A, A, B2, 1e-6f, NULL, NULL, A, 1 << 30, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_noncausal(SVLA_BF16, 1, 2, 64, 32, MIS, A, A, B2, 1e-6f, NULL, NULL, A, 1 << 30, NULL) == SVLA_ERR_ALIGN);
    EXPECT(svla_block_causal(SVLA_BF16, 1, 2, 2, 64, 48, A, A, A, B2, NULL, NULL, NULL, NULL, NULL, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_UNSUPPORTED);
    EXPECT(svla_block_causal(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, B2, F, NULL, NULL, NULL, NULL, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_block_causal(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, B2, NULL, NULL, NULL, NULL, NULL, -1.f, A, 1 << 30, NULL) == SVLA_ERR_VALUE);
    EXPECT(svla_block_causal(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, B2, NULL, NULL, NULL, NULL, NULL, 1e-6f, A, 16, NULL) == SVLA_ERR_WORKSPACE);
    EXPECT(svla_block_causal(SVLA_BF16, 1, 2, 1, 1 << 26, 32, A, A, A, B2, NULL, NULL, NULL, NULL, NULL, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_SHAPE);
    {
        svla_rope odd = {3, 0, 0, 1, 1, 0, 1e4f}, neg = {2, 2, 2, 1, 1, -1, 1e4f}, big = {8, 12, 12, 1000, 1000, 0, 1e4f};
        EXPECT(svla_block_causal(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, B2, NULL, NULL, NULL, NULL, &odd, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_VALUE);
        EXPECT(svla_block_causal(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, B2, NULL, NULL, NULL, NULL, &neg, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_VALUE);
        EXPECT(svla_block_causal(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, B2, NULL, NULL, NULL, NULL, &big, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_UNSUPPORTED);
    }
    EXPECT(svla_block_causal_gated(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, B2, NULL, NULL, NULL, NULL, NULL, NULL, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_block_step(SVLA_BF16, 1, 2, 64, 32, A, A, A, B2, NULL, NULL, NULL, NULL, NULL, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_block_step_gated(SVLA_BF16, 1, 2, 64, 32, A, A, A, B2, NULL, NULL, F, F, NULL, NULL, 1e-6f, A, 1 << 30, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_block_step_noalloc(SVLA_BF16, 1, 2, 64, 32, A, A, A, B2, NULL, NULL, NULL, NULL, NULL, NULL, 1e-6f, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_block_step_noalloc(SVLA_BF16, 1, 2, 64, 32, A, A, A, B2, NULL, NULL, F, F, NULL, NULL, -2.f, NULL) == SVLA_ERR_VALUE);
    EXPECT(svla_block_step_noalloc(SVLA_BF16, 64, 64, 2048, 128, A, A, A, B2, NULL, NULL, F, F, NULL, NULL, 1e-6f, NULL) == SVLA_ERR_WORKSPACE);
    EXPECT(svla_state_build(SVLA_BF16, 1, 2, 2, 64, 32, A, A, NULL, NULL, NULL, NULL, 0, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_state_scan(1, 2, 2, 32, F, F, NULL, F, NULL, F, F, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_apply(SVLA_BF16, 1, 2, 2, 64, 32, A, F, F, NULL, 1e-6f, B2, NULL, 0, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_temporal_conv(SVLA_BF16, 1, 2, 3, 4, 12, A, B2, F, NULL, NULL, NULL, NULL) == SVLA_ERR_UNSUPPORTED);
    EXPECT(svla_temporal_conv(SVLA_BF16, 1, 2, 3, 4, 16, A, (char *)A + 64, F, NULL, NULL, NULL, NULL) == SVLA_ERR_VALUE);
    EXPECT(svla_temporal_conv(SVLA_FP8, 1, 2, 3, 4, 16, A, B2, F, NULL, NULL, NULL, NULL) == SVLA_ERR_DTYPE);
    EXPECT(svla_block_causal_backward(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, A, NULL, NULL, NULL, NULL, 1e-6f,
                                      A, B2, (char *)B2 + (1 << 20), NULL, NULL, NULL, (char *)B2 + (2 << 20), 1 << 30, NULL) == SVLA_ERR_VALUE);
    EXPECT(svla_block_causal_backward(SVLA_FP8, 1, 2, 2, 64, 32, A, A, A, A, NULL, NULL, NULL, NULL, 1e-6f,
                                      B2, B2, B2, NULL, NULL, NULL, A, 1 << 30, NULL) == SVLA_ERR_UNSUPPORTED);
    EXPECT(svla_block_causal_backward(SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, NULL, NULL, NULL, NULL, NULL, 1e-6f,
                                      B2, B2, B2, NULL, NULL, NULL, A, 1 << 30, NULL) == SVLA_ERR_NULL);
    EXPECT(svla_set_timing_events(NULL, -1) == SVLA_OK);
    EXPECT(svla_set_timing_events((void *const *)&A, -1) == SVLA_ERR_VALUE);
    printf("libsvla host side under sanitizers: %s\n", fails ? "FAILED" : "clean");
    return fails != 0;
}
