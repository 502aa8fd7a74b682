/*
 * C driver of libgdr's host side, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer against a host-only build of the library (no
 * device code).  Every entry point is called through the C ABI with invalid
 * arguments (each must be rejected with its status before any HIP call) and,
 * on a host without a GPU, with valid arguments, which must come back as
 * GDR_ERR_HIP instead of crashing.  Exit status: 0 pass, 1 a check failed,
 * 77 skipped (a GPU is visible: the valid calls would launch kernels on the
 * fake addresses used here).
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "gdr.h"

/* From the HIP runtime (C linkage): the number of visible devices. */
extern int hipGetDeviceCount(int* count);

static int failures = 0;

#define EXPECT(call, want)                                                            \
    do {                                                                              \
        int got_ = (call);                                                            \
        if (got_ != (want)) {                                                         \
            fprintf(stderr, "line %d: %s = %d, expected %d\n", __LINE__, #call, got_, \
                    (want));                                                          \
            ++failures;                                                               \
        }                                                                             \
    } while (0)

/* Fake, non-NULL, 4 KiB-aligned addresses: never dereferenced on the host. */
static void* fake(int i) { return (void*)(uintptr_t)(0x100000u * (unsigned)(i + 1)); }

int main(void) {
    int ndev = 0;
    const int hip_status = hipGetDeviceCount(&ndev);
    if (hip_status == 0 && ndev > 0) {
        printf("a GPU is visible: skipped\n");
        return 77;
    }
    void* p[16];
    for (int i = 0; i < 16; ++i) p[i] = fake(i);
    const float* fa = (const float*)p[3];
    const float* fb = (const float*)p[4];

    /* status strings, including codes the library does not know */
    for (int s = -10; s <= 2; ++s)
        if (!gdr_status_string(s)) ++failures;
    EXPECT(gdr_abi_version(), GDR_ABI_VERSION);

    /* decode: enums, shapes, head sizes, pointers, alignment, zero size */
    EXPECT(gdr_decode_step(2, 1, 2, 3, 128, 128, 1.f, p[0], p[1], p[2], fa, fb, p[5], p[6], 0),
           GDR_ERR_BAD_ENUM);
    EXPECT(gdr_decode_step(0, 1, -1, 3, 128, 128, 1.f, p[0], p[1], p[2], fa, fb, p[5], p[6], 0),
           GDR_ERR_BAD_SHAPE);
    EXPECT(gdr_decode_step(0, 1, INT_MAX, INT_MAX, 128, 128, 1.f, p[0], p[1], p[2], fa, fb, p[5],
                           p[6], 0),
           GDR_ERR_BAD_SHAPE);
    EXPECT(gdr_decode_step(0, 1, 2, 3, 96, 128, 1.f, p[0], p[1], p[2], fa, fb, p[5], p[6], 0),
           GDR_ERR_UNSUPPORTED);
    EXPECT(gdr_decode_step(0, 1, 2, 3, 128, 128, 1.f, 0, p[1], p[2], fa, fb, p[5], p[6], 0),
           GDR_ERR_NULL_PTR);
    EXPECT(gdr_decode_step(1, 1, 2, 3, 128, 128, 1.f, p[0], p[1], p[2], fa + 1, fb, p[5], p[6], 0),
           GDR_ERR_MISALIGNED);
    EXPECT(gdr_decode_step(0, 1, 0, 3, 128, 128, 1.f, 0, 0, 0, 0, 0, 0, 0, 0), GDR_OK);
    EXPECT(gdr_decode_step_ex(0, 1, GDR_SCHED_SPLIT, 2, 3, 128, 128, 1.f, p[0], p[1], p[2], fa, fb,
                              p[5], p[6], 0),
           GDR_ERR_BAD_ENUM);
    EXPECT(gdr_decode_multi(0, 1, 2, 65, 3, 128, 128, 1.f, p[0], p[1], p[2], fa, fb, p[5], p[6], 0, 0),
           GDR_ERR_UNSUPPORTED);
    /* kept states overlapping the state */
    EXPECT(gdr_decode_multi(0, 1, 2, 4, 3, 128, 128, 1.f, p[0], p[1], p[2], fa, fb, p[5], p[6],
                            (float*)p[5], 0),
           GDR_ERR_ALIAS);

    /* prefill: flags, schedules, chunk, workspace, aliasing */
    EXPECT(gdr_chunk_prefill_ex(0, 1, GDR_SCHED_FUSED | GDR_SCHED_SPLIT, 2, 70, 3, 128, 128, 64,
                                1.f, p[0], p[1], p[2], fa, fb, 0, p[7], p[8], 0, 0, 0),
           GDR_ERR_BAD_ENUM);
    EXPECT(gdr_chunk_prefill_ex(1, 1, GDR_SCHED_FUSED, 2, 70, 3, 128, 128, 64, 1.f, p[0], p[1],
                                p[2], fa, fb, 0, p[7], p[8], 0, 0, 0),
           GDR_ERR_UNSUPPORTED);
    EXPECT(gdr_chunk_prefill(0, 1, 2, 70, 3, 128, 128, 32, 1.f, p[0], p[1], p[2], fa, fb, 0, p[7],
                             p[8], 0, 0, 0),
           GDR_ERR_UNSUPPORTED);
    EXPECT(gdr_chunk_prefill(1, 1, 2, 70, 3, 128, 128, 64, 1.f, p[0], p[1], p[2], fa, fb, 0, p[7],
                             p[8], 0, 0, 0),
           GDR_ERR_WORKSPACE);
    EXPECT(gdr_chunk_prefill(0, 1, INT_MAX, INT_MAX, INT_MAX, 128, 128, 64, 1.f, p[0], p[1], p[2],
                             fa, fb, 0, p[7], p[8], 0, 0, 0),
           GDR_ERR_BAD_SHAPE);
    {
        float* s_out = (float*)p[7];
        EXPECT(gdr_chunk_prefill(0, 1, 2, 70, 3, 128, 128, 64, 1.f, p[0], p[1], p[2], fa, fb,
                                 s_out + 4, s_out, p[8], 0, 0, 0),
               GDR_ERR_ALIAS);
    }
    if (gdr_chunk_prefill_workspace_bytes(0, 1, INT_MAX, INT_MAX, INT_MAX, 128, 128, 64) != 0)
        ++failures;
    if (gdr_chunk_prefill_workspace_bytes_ex(1, 1, 0, 1, 32768, 32, 128, 128, 64) == 0) ++failures;
    if (gdr_chunk_prefill_varlen_workspace_bytes_ex(0, 1, GDR_SCHED_SPLIT | GDR_PRO_L2NORM_QK, 4,
                                                    64, 2, 64, 64, 64) != 0)
        ++failures;
    EXPECT(gdr_chunk_prefill_varlen(0, 1, 2, 100, 70, 3, 128, 128, 64, 1.f, p[0], p[1], p[2], fa,
                                    fb, 0, p[6], 0, p[7], 4, p[8], 0, 0, 0),
           GDR_ERR_NULL_PTR);

    /* backward */
    EXPECT(gdr_chunk_backward(0, 1, 1, 64 * (1 << 22), 1, 128, 128, 64, 1.f, p[0], p[1], p[2], fa,
                              fb, 0, p[5], 0, p[6], p[7], p[8], (float*)p[9], (float*)p[10], 0,
                              p[11], (size_t)1 << 40, 0),
           GDR_ERR_BAD_SHAPE);
    if (gdr_chunk_backward_workspace_bytes(0, 1, INT_MAX, INT_MAX, 1, 128, 128, 64) != 0) ++failures;
    if (gdr_chunk_backward_workspace_bytes_ranged(0, 1, INT_MAX, INT_MAX, 1, 128, 128, 64, 1) != 0)
        ++failures;
    if (gdr_chunk_backward_workspace_bytes_ranged(0, 1, 1, 130, 2, 64, 64, 64, 0) != 0) ++failures;

    /* valid calls on a host without a GPU: the runtime rejects them */
    EXPECT(gdr_decode_step(0, 1, 2, 3, 128, 128, 1.f, p[0], p[1], p[2], fa, fb, p[5], p[6], 0),
           GDR_ERR_HIP);
    EXPECT(gdr_decode_multi(1, 1, 2, 4, 3, 64, 64, 1.f, p[0], p[1], p[2], fa, fb, p[5], p[6], 0, 0),
           GDR_ERR_HIP);
    EXPECT(gdr_chunk_prefill(0, 1, 2, 70, 3, 128, 128, 64, 1.f, p[0], p[1], p[2], fa, fb, 0, p[7],
                             p[8], 0, 0, 0),
           GDR_ERR_HIP);
    EXPECT(gdr_chunk_prefill(0, 0, 2, 70, 3, 32, 32, 64, 1.f, p[0], p[1], p[2], fa, fb, 0, p[7],
                             p[8], 0, 0, 0),
           GDR_ERR_HIP);
    {
        const size_t need = gdr_chunk_prefill_workspace_bytes(1, 1, 2, 70, 3, 128, 128, 64);
        EXPECT(gdr_chunk_prefill(1, 1, 2, 70, 3, 128, 128, 64, 1.f, p[0], p[1], p[2], fa, fb, 0,
                                 p[7], p[8], p[9], need, 0),
               GDR_ERR_HIP);
    }
    EXPECT(gdr_chunk_prefill(0, 1, 2, 0, 3, 128, 128, 64, 1.f, 0, 0, 0, 0, 0, 0, p[7], 0, 0, 0, 0),
           GDR_ERR_HIP); /* T == 0: the state copy kernel */
    /* the call without a workspace: its scratch lookup fails without a GPU */
    EXPECT(gdr_chunk_prefill_noalloc(1, 1, 0, 2, 70, 3, 128, 128, 64, 1.f, p[0], p[1], p[2], fa, fb,
                                     0, p[7], p[8], 0),
           GDR_ERR_HIP);
    EXPECT(gdr_chunk_prefill_noalloc(1, 1, 0, 1, 70, 1446, 128, 128, 64, 1.f, p[0], p[1], p[2], fa,
                                     fb, 0, p[7], p[8], 0),
           GDR_ERR_SCRATCH);
    {
        const size_t need = gdr_chunk_backward_workspace_bytes(1, 0, 1, 130, 2, 64, 64, 64);
        EXPECT(gdr_chunk_backward(1, 0, 1, 130, 2, 64, 64, 64, 1.f, p[0], p[1], p[2], fa, fb, 0,
                                  p[5], 0, p[6], p[7], p[8], (float*)p[9], (float*)p[10], 0,
                                  p[11], need, 0),
               GDR_ERR_HIP);
        /* the same in ranges of one chunk (the ranged host driver) */
        const size_t one = gdr_chunk_backward_workspace_bytes_ranged(1, 0, 1, 130, 2, 64, 64, 64, 1);
        if (!(one > 0 && one < need)) ++failures;
        EXPECT(gdr_chunk_backward(1, 0, 1, 130, 2, 64, 64, 64, 1.f, p[0], p[1], p[2], fa, fb, 0,
                                  p[5], 0, p[6], p[7], p[8], (float*)p[9], (float*)p[10], 0,
                                  p[11], one, 0),
               GDR_ERR_HIP);
    }
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("all checks passed\n");
    return 0;
}
