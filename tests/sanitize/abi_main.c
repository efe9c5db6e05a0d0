/*
 * Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * library's host code (tests/test_sanitizers_cpu.py): every entry point of
 * include/grkan.h is called with arguments it must reject -- null, misaligned
 * or overlapping pointers, bad shapes, sizes near the int64 limits, unknown
 * flags and degrees -- and the host-only queries are called over many
 * shapes.  None of these calls may reach the HIP runtime (validation precedes
 * every HIP call), so the run needs no GPU; the fake device addresses below
 * are never dereferenced.  Exit status 0 = every call returned the expected
 * status; a sanitizer report aborts with a non-zero status.
 */
#include <stdint.h>
#include <stdio.h>

#include "grkan.h"

static int failures = 0;
#define EXPECT(call, st)                                                                  \
    do {                                                                                  \
        grkan_status_t got_ = (call);                                                     \
        if (got_ != (st)) {                                                               \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call,   \
                    (int)got_, (int)(st));                                                \
            ++failures;                                                                   \
        }                                                                                 \
    } while (0)

#define P(off) ((void *)(uintptr_t)(0x100000u + (off)))
#define F(off) ((float *)(uintptr_t)(0x100000u + (off)))

int main(void)
{
    const grkan_status_t INV = GRKAN_ERR_INVALID_ARG, UNS = GRKAN_ERR_UNSUPPORTED;
    for (int s = -2; s < 6; ++s)
        if (!grkan_status_string((grkan_status_t)s)) ++failures;

    /* host-only queries over many shapes, including near-overflow sizes */
    const int64_t rows[] = {0, 1, 15, 16, 17, 1001, 201728, (int64_t)1 << 40, INT64_MAX};
    const int64_t ds[] = {1, 8, 40, 64, 768, 3072, 65536 * 4, (int64_t)1 << 40};
    const int32_t gs[] = {1, 8, 768, 65536};
    for (unsigned i = 0; i < sizeof rows / sizeof rows[0]; ++i)
        for (unsigned j = 0; j < sizeof ds / sizeof ds[0]; ++j)
            for (unsigned k = 0; k < sizeof gs / sizeof gs[0]; ++k)
                for (int io = 0; io < 3; ++io)
                    for (uint32_t fl = 0; fl < 9; ++fl) {
                        (void)grkan_backward_workspace_size(rows[i], ds[j], gs[k], (grkan_dtype_t)io, fl);
                        (void)grkan_pau_backward_workspace_size(rows[i], ds[j], gs[k], 7, 6, (grkan_dtype_t)io, fl);
                    }
    for (int m = -1; m < 17; ++m)
        for (int n = -1; n < 17; ++n) (void)grkan_pau_supported(m, n);
    (void)grkan_layer_backward_workspace_size(201728, 768, 3072, 8);
    (void)grkan_layer_backward_workspace_size(INT64_MAX, 768, 3072, 8);
    (void)grkan_chebykan_backward_workspace_size(201728, 768, 768, 7);
    (void)grkan_chebykan_backward_workspace_size(INT64_MAX, 1 << 30, 768, 7);

    /* forward */
    EXPECT(grkan_forward(NULL, P(0x100000), F(0x200000), F(0x300000), 4, 64, 8, GRKAN_F32, 0), INV);
    EXPECT(grkan_forward(P(4), P(0x100000), F(0x200000), F(0x300000), 4, 64, 8, GRKAN_F32, 0), UNS);
    EXPECT(grkan_forward(P(0), P(16), F(0x200000), F(0x300000), 4, 64, 8, GRKAN_F32, 0), INV);
    EXPECT(grkan_forward(P(0), P(0x100000), F(0x200000), F(0x300000), 4, 66, 8, GRKAN_F32, 0), INV);
    EXPECT(grkan_forward(P(0), P(0x100000), F(0x200000), F(0x300000), INT64_MAX, 64, 8, GRKAN_F32, 0), INV);
    EXPECT(grkan_forward(P(0), P(0x100000), F(0x200000), F(0x300000), 4, 64, 8, (grkan_dtype_t)7, 0), INV);
    EXPECT(grkan_forward(NULL, NULL, F(0x200000), F(0x300000), 0, 64, 8, GRKAN_F32, 0), GRKAN_OK);

    /* backward, every flag word and bad workspaces */
    for (uint32_t fl = 3; fl < 64; ++fl)
        if (fl != 4)
            EXPECT(grkan_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), F(0x500000),
                                  F(0x600000), 4, 64, 8, GRKAN_F32, fl, P(0x700000), 1 << 20, 0), INV);
    EXPECT(grkan_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), F(0x500000), F(0x600000),
                          4, 64, 8, GRKAN_F32, 1, P(0x700000), 100, 0), INV);
    EXPECT(grkan_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), F(0x500000), F(0x600000),
                          4, 64, 8, GRKAN_F32, 0, P(0x400000 - 64), 1 << 20, 0), INV);
    EXPECT(grkan_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(16), F(0x500000), F(0x600000),
                          4, 64, 8, GRKAN_F32, 0, P(0x700000), 1 << 20, 0), INV);
    EXPECT(grkan_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), F(0x500001), F(0x600000),
                          4, 64, 8, GRKAN_F32, 0, P(0x700000), 1 << 20, 0), UNS);
    EXPECT(grkan_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), F(0x500000), F(0x600000),
                          (int64_t)1 << 62, 1 << 20, 8, GRKAN_BF16, 0, P(0x700000), 1 << 20, 0), INV);

    /* PAU family and the probe */
    EXPECT(grkan_pau_forward(P(0), P(0x100000), F(0x200000), F(0x300000), 4, 64, 8, 9, 9, GRKAN_F32, 0), UNS);
    EXPECT(grkan_pau_forward(P(0), P(0x100000), F(0x200000), F(0x300000), 4, 64, 8, -1, 2, GRKAN_F32, 0), INV);
    EXPECT(grkan_pau_backward(P(0), P(0x100000), F(0x200000), NULL, P(0x400000), F(0x500000), F(0x600000), 4,
                              64, 8, 3, 2, GRKAN_F32, 0, P(0x700000), 1 << 20, 0), INV);
    EXPECT(grkan_pau_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), F(0x500000),
                              F(0x600000), 4, 64, 8, 3, 2, GRKAN_F32, GRKAN_NAIVE_ATOMIC, P(0x700000), 1 << 20, 0),
           UNS);
    EXPECT(grkan_inflated_forward(P(0), P(0x100000), F(0x200000), F(0x300000), 4, 64, 8, GRKAN_F32, 3, 0), INV);
    EXPECT(grkan_inflated_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), F(0x500000),
                                   F(0x600000), 4, 40, 8, GRKAN_F32, 0, 2, P(0x700000), 1 << 20, 0), UNS);
    EXPECT(grkan_stream_probe(P(0), P(0x1000), P(16), 64, 0), INV);
    EXPECT(grkan_stream_probe(P(0), P(0x1000), P(0x2000), 24, 0), UNS);
    EXPECT(grkan_stream_probe(NULL, NULL, NULL, 0, 0), GRKAN_OK);
    EXPECT(grkan_backward_noalloc(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), F(0x500000),
                                  F(0x600000), 5 * 201728, 3072, 8, GRKAN_BF16, 0), UNS);
    EXPECT(grkan_backward_noalloc(P(0), P(0x100000), F(0x200000), F(0x300000), P(16), F(0x500000),
                                  F(0x600000), 4, 64, 8, GRKAN_F32, 0), INV);
    grkan_launch_t launch;
    EXPECT(grkan_query_launch(4, 64, 8, GRKAN_F32, 3, &launch), INV);
    EXPECT(grkan_query_launch(4, 64, 8, GRKAN_F32, 0, NULL), INV);

    /* the layer and the Chebyshev-KAN layer */
    EXPECT(grkan_layer_forward(P(0), F(0x200000), F(0x300000), P(0x400000), P(0x500000), 4, 100, 64, 8, 0), UNS);
    EXPECT(grkan_layer_forward(P(0), F(0x200000), F(0x300000), P(0x400000), P(16), 4, 64, 64, 8, 0), INV);
    EXPECT(grkan_linear_forward(P(0), P(0x400000), P(0x500000), -1, 64, 64, 0), INV);
    EXPECT(grkan_layer_backward(P(0), P(0x100000), F(0x200000), F(0x300000), P(0x400000), P(0x500000),
                                F(0x600000), F(0x700000), F(0x800000), 4, 64, 100, 8, P(0x900000), 1 << 20, 0),
           UNS);
    EXPECT(grkan_chebykan_forward(P(0), P(0x400000), P(0x500000), 4, 64, 64, 6, 0), UNS);
    EXPECT(grkan_chebykan_backward(P(0), P(0x100000), P(0x400000), P(0x500000), F(0x600000), 4, 64, 64, 7,
                                   P(0x900000), 100, 0), INV);
    if (failures) {
        fprintf(stderr, "%d calls returned an unexpected status\n", failures);
        return 1;
    }
    puts("ABI sanitizer run: ok");
    return 0;
}
