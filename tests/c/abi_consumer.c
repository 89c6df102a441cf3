/* A plain C99 consumer of include/mi_attn.h, linked against libmi_attn.so.
 * It runs without a GPU: every call here is either a query of the library
 * or an argument error that the library reports before any HIP call, so no
 * pointer below is ever dereferenced.  Exit status: number of failures. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "mi_attn.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
    if (got != want) {
        printf("FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

int main(void) {
    void* q = (void*)0x10000;
    void* k = (void*)0x20000;
    void* v = (void*)0x30000;
    void* o = (void*)0x40000;
    float* lse = (float*)0x50000;

    expect("version", mi_attn_version(), MI_ATTN_ABI_VERSION);
    expect("last hip error", mi_attn_last_hip_error(), 0);
    if (mi_attn_status_string(MI_ATTN_ERR_SHAPE) == NULL ||
        strstr(mi_attn_status_string(MI_ATTN_ERR_SHAPE), "MI_ATTN_ERR_SHAPE") == NULL) {
        printf("FAIL status string\n");
        ++failures;
    }

    /* forward: Hq not a multiple of Hkv, an unsupported head_dim, a wrong
     * dtype, a NULL q, an unaligned pointer, a NaN scale */
    expect("hq % hkv", mi_attn_fwd(q, k, v, o, lse, MI_ATTN_F16, MI_ATTN_F16, 1, 3, 2, 16, 16, 64,
                                   NULL, NULL, NULL, NULL, NULL, NULL, 0.125f, 0, NULL),
           MI_ATTN_ERR_SHAPE);
    expect("head_dim 96", mi_attn_fwd(q, k, v, o, lse, MI_ATTN_BF16, MI_ATTN_BF16, 1, 2, 2, 16, 16,
                                      96, NULL, NULL, NULL, NULL, NULL, NULL, 0.1f, 0, NULL),
           MI_ATTN_ERR_UNSUPPORTED);
    expect("f32 input", mi_attn_fwd(q, k, v, o, lse, MI_ATTN_F32, MI_ATTN_F32, 1, 2, 2, 16, 16, 64,
                                    NULL, NULL, NULL, NULL, NULL, NULL, 0.125f, 0, NULL),
           MI_ATTN_ERR_DTYPE);
    expect("null q", mi_attn_fwd(NULL, k, v, o, lse, MI_ATTN_F16, MI_ATTN_F16, 1, 2, 2, 16, 16, 64,
                                 NULL, NULL, NULL, NULL, NULL, NULL, 0.125f, 1, NULL),
           MI_ATTN_ERR_NULL);
    expect("unaligned k", mi_attn_fwd(q, (char*)k + 8, v, o, lse, MI_ATTN_F16, MI_ATTN_F16, 1, 2,
                                      2, 16, 16, 64, NULL, NULL, NULL, NULL, NULL, NULL, 0.125f, 0,
                                      NULL),
           MI_ATTN_ERR_LAYOUT);
    expect("nan scale", mi_attn_fwd(q, k, v, o, lse, MI_ATTN_F16, MI_ATTN_F16, 1, 2, 2, 16, 16, 64,
                                    NULL, NULL, NULL, NULL, NULL, NULL, (float)NAN, 0, NULL),
           MI_ATTN_ERR_ARG);
    {
        /* a row stride below head_dim (an expanded view) */
        const mi_attn_strides_t bad = {0, 64, 0};
        expect("row stride 0", mi_attn_fwd(q, k, v, o, lse, MI_ATTN_F16, MI_ATTN_F16, 1, 2, 2, 16,
                                           16, 64, NULL, &bad, NULL, NULL, NULL, NULL, 0.125f, 0,
                                           NULL),
               MI_ATTN_ERR_LAYOUT);
    }
    /* an empty batch is a no-op that succeeds, even with NULL tensors */
    expect("empty batch", mi_attn_fwd(NULL, NULL, NULL, NULL, NULL, MI_ATTN_F16, MI_ATTN_F16, 0, 2,
                                      2, 16, 16, 64, NULL, NULL, NULL, NULL, NULL, NULL, 0.125f, 0,
                                      NULL),
           MI_ATTN_OK);
    /* select: an unknown kernel; dropout: p = 1 */
    expect("unknown kernel", mi_attn_fwd_select(q, k, v, o, lse, MI_ATTN_F16, MI_ATTN_F16, 1, 2, 2,
                                                16, 16, 64, NULL, NULL, NULL, NULL, NULL, NULL,
                                                0.125f, 0, NULL, (mi_attn_kernel_t)7, -1),
           MI_ATTN_ERR_ARG);
    expect("dropout 1", mi_attn_fwd_dropout(q, k, v, o, lse, MI_ATTN_F16, MI_ATTN_F16, 1, 2, 2, 16,
                                            16, 64, NULL, NULL, NULL, NULL, NULL, NULL, 0.125f, 0,
                                            1.0, 7u, NULL),
           MI_ATTN_ERR_ARG);
    /* decode plan queries */
    if (mi_attn_decode_splits(8, 32, 8, 1, 8192, 128, 0) < 1) {
        printf("FAIL decode splits\n");
        ++failures;
    }
    if (mi_attn_decode_workspace_size(8, 32, 8, 1, 8192, 128, 0) == 0) {
        printf("FAIL decode workspace size\n");
        ++failures;
    }
    if (mi_attn_decode_noalloc_max_bytes() == 0) {
        printf("FAIL noalloc max bytes\n");
        ++failures;
    }
    /* rotary: a rotary dimension that is not a multiple of 16; Q and K the
     * same tensor */
    expect("rotary dim 24", mi_attn_rotary(q, MI_ATTN_BF16, 1, 4, 100, 128, NULL, NULL, NULL, 0, 24,
                                           10000.0, 0, NULL),
           MI_ATTN_ERR_UNSUPPORTED);
    expect("rotary qk same", mi_attn_rotary_qk(q, q, MI_ATTN_BF16, 1, 4, 2, 100, 128, NULL, NULL,
                                               NULL, NULL, 0, 128, 10000.0, 0, NULL),
           MI_ATTN_ERR_LAYOUT);
    expect("last hip error still 0", mi_attn_last_hip_error(), 0);

    if (failures == 0) printf("c consumer: all checks passed\n");
    return failures;
}
