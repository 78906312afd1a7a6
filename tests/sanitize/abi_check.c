/*
 * Calls every entry point of include/bdssm.h with argument sets that validation must
 * reject (NULL pointers, bad shapes and dtypes, misaligned pointers, overlapping outputs,
 * missing workspace), and the workspace and size queries, so that a build of the host
 * library with AddressSanitizer and UndefinedBehaviorSanitizer checks the host-side
 * validation code. Nothing here reaches a kernel or needs a GPU. Exits non-zero if a call
 * returns an unexpected status.
 */
#include <stdint.h>
#include <stdio.h>

#include "bdssm.h"

#define FAKE ((uintptr_t)1 << 20)
#define P(v) ((void *)(uintptr_t)(v))
#define EXPECT(call, want)                                                           \
    do {                                                                             \
        const int rc_ = (int)(call);                                                 \
        if (rc_ != (want)) {                                                         \
            fprintf(stderr, "%s: got %d (%s), want %d\n", #call, rc_, bdssm_status_str(rc_), (int)(want)); \
            return 1;                                                                \
        }                                                                            \
    } while (0)

int main(void)
{
    bdssm_dims d = {1, 4, 16, 16, 1, BDSSM_F32, BDSSM_F32};
    bdssm_dims bf = {1, 4, 64, 128, 1, BDSSM_BF16, BDSSM_F32};
    const uintptr_t base = (uintptr_t)1 << 40;
    bdssm_seq s = {P(base), P(base + (1ull << 32)), P(base + (2ull << 32)), P(base + (3ull << 32))};
    bdssm_seq r = {P(base + (4ull << 32)), P(base + (5ull << 32)), P(base + (6ull << 32)), P(base + (7ull << 32))};
    const float *A = (const float *)P(FAKE), *D = (const float *)P(FAKE + 256), *Ar = (const float *)P(FAKE + 512);
    float *h = (float *)P(base + (8ull << 32));
    void *y = P(base + (9ull << 32)), *ws = P(base + (10ull << 32));
    bdssm_dims bad = d;
    bad.ngroups = 3;

    EXPECT(bdssm_abi_version(), BDSSM_ABI_VERSION);
    for (int st = -1; st <= 9; ++st)
        if (!bdssm_status_str(st))
            return 1;
    /* prefix scan */
    EXPECT(bdssm_prefix_scan(NULL, 64, 64, &s, A, D, NULL, NULL, NULL, h, NULL, 0, NULL), BDSSM_ERR_NULL);
    EXPECT(bdssm_prefix_scan(&bad, 64, 64, &s, A, D, NULL, NULL, NULL, h, NULL, 0, NULL), BDSSM_ERR_SHAPE);
    EXPECT(bdssm_prefix_scan(&d, -1, 64, &s, A, D, NULL, NULL, NULL, h, NULL, 0, NULL), BDSSM_ERR_SHAPE);
    EXPECT(bdssm_prefix_scan(&d, 64, 48, &s, A, D, NULL, NULL, NULL, h, NULL, 0, NULL), BDSSM_ERR_UNSUPPORTED);
    EXPECT(bdssm_prefix_scan(&d, 64, 64, &s, A, D, NULL, P(base + 2), NULL, h, NULL, 0, NULL), BDSSM_ERR_ALIGN);
    EXPECT(bdssm_prefix_scan(&d, 64, 64, &s, A, D, NULL, (void *)s.x, NULL, h, NULL, 0, NULL), BDSSM_ERR_ALIAS);
    EXPECT(bdssm_prefix_scan(&bf, 8192, 256, &s, A, D, NULL, y, NULL, h, NULL, 0, NULL), BDSSM_ERR_WORKSPACE);
    EXPECT(bdssm_prefix_scan_static(NULL, 64, 64, &s, A, D, NULL, NULL, NULL, h, NULL), BDSSM_ERR_NULL);
    if (bdssm_prefix_scan_workspace(&bad, 64, 64, 1, 1) != SIZE_MAX || bdssm_prefix_scan_workspace(&bf, 8192, 256, 1, 0) == 0)
        return 1;
    /* block steps */
    EXPECT(bdssm_block_step(&d, 16, NULL, &s, &r, A, D, y, NULL), BDSSM_ERR_NULL);
    EXPECT(bdssm_block_step(&d, 257, h, &s, &r, A, D, y, NULL), BDSSM_ERR_UNSUPPORTED);
    EXPECT(bdssm_block_step(&d, 16, h, &s, &r, A, D, (void *)s.x, NULL), BDSSM_ERR_ALIAS);
    EXPECT(bdssm_block_step_ex(&d, 16, h, &s, &r, A, D, NULL, NULL, y, NULL), BDSSM_ERR_NULL);
    EXPECT(bdssm_block_step_ex(&d, 16, h, &s, &r, A, D, (const float *)P(FAKE + 4), NULL, y, NULL), BDSSM_ERR_ALIGN);
    EXPECT(bdssm_block_step_ops(&d, 16, h, &s, &r, A, D, Ar, NULL, y, NULL), BDSSM_ERR_UNSUPPORTED);
    bdssm_step_params prm = {A, D, NULL, NULL, 0};
    EXPECT(bdssm_block_step_variant(&d, 16, h, 7, &s, &r, &prm, y, NULL), BDSSM_ERR_UNSUPPORTED);
    EXPECT(bdssm_block_step_variant(&d, 16, h, BDSSM_STATE_OPS, &s, &r, &prm, y, NULL), BDSSM_ERR_UNSUPPORTED);
    EXPECT(bdssm_block_step_variant(&d, 16, h, BDSSM_STATE_F32, &s, &r, NULL, y, NULL), BDSSM_ERR_NULL);
    prm.skip_per_channel = 2;
    EXPECT(bdssm_block_step_variant(&d, 16, h, BDSSM_STATE_BF16, &s, &r, &prm, y, NULL), BDSSM_ERR_UNSUPPORTED);
    /* state encodings */
    if (bdssm_state_ops_bytes(&d) != SIZE_MAX || bdssm_state_bf16_bytes(&d) != 4 * 16 * 16 * 2)
        return 1;
    EXPECT(bdssm_state_ops(&d, h, y, NULL), BDSSM_ERR_UNSUPPORTED);
    EXPECT(bdssm_state_bf16(&d, h, P(base + (8ull << 32) + 512), NULL), BDSSM_ERR_ALIAS);
    /* commits */
    EXPECT(bdssm_commit(&d, 16, &s, A, D, NULL, NULL, NULL), BDSSM_ERR_NULL);
    EXPECT(bdssm_commit(&d, -1, &s, A, D, h, NULL, NULL), BDSSM_ERR_SHAPE);
    EXPECT(bdssm_commit(&d, 16, &s, A, D, (float *)s.x, NULL, NULL), BDSSM_ERR_ALIAS);
    EXPECT(bdssm_commit_refresh(&d, 16, &s, A, D, h, y, BDSSM_STATE_OPS, NULL, NULL), BDSSM_ERR_UNSUPPORTED);
    EXPECT(bdssm_commit_refresh(&d, 16, &s, A, D, h, NULL, BDSSM_STATE_BF16, NULL, NULL), BDSSM_ERR_NULL);
    /* full window */
    EXPECT(bdssm_full_window(&d, 64, 64, &s, &r, A, D, NULL, NULL, y, NULL, 0, NULL), BDSSM_ERR_NULL);
    EXPECT(bdssm_full_window(&d, 64, 64, &s, &r, A, D, Ar, NULL, (void *)s.x, NULL, 0, NULL), BDSSM_ERR_ALIAS);
    EXPECT(bdssm_full_window(&bf, 8192, 256, &s, &r, A, D, Ar, NULL, y, NULL, 0, NULL), BDSSM_ERR_WORKSPACE);
    /* convolution state */
    bdssm_conv_params cp = {4, 1, (const float *)P(FAKE + 1024), NULL};
    bdssm_conv_params cbad = {5, 1, (const float *)P(FAKE + 1024), NULL};
    EXPECT(bdssm_conv(&d, 10, &cbad, 0, NULL, &s, &r, NULL, NULL), BDSSM_ERR_UNSUPPORTED);
    EXPECT(bdssm_conv(&d, 10, &cp, 1, P(base), &s, &r, NULL, NULL), BDSSM_ERR_SHAPE);
    EXPECT(bdssm_block_step_conv(&d, 16, &cp, &cp, h, NULL, &s, &r, A, D, NULL, NULL, y, ws, 1 << 20, NULL),
           BDSSM_ERR_NULL);
    EXPECT(bdssm_commit_conv(&d, 16, &cp, &s, A, D, h, P(base + (11ull << 32)), NULL, NULL, 0, NULL),
           BDSSM_ERR_WORKSPACE);
    if (bdssm_conv_workspace(&d, -1) != SIZE_MAX)
        return 1;
    /* decode graph and launch override */
    bdssm_decode_graph *g = (bdssm_decode_graph *)P(1);
    EXPECT(bdssm_decode_graph_create(&d, 16, 1, h, NULL, &s, &r, A, D, &y, NULL, NULL, NULL, &g), BDSSM_ERR_NULL);
    if (g != NULL)
        return 1;
    EXPECT(bdssm_decode_graph_launch(NULL, NULL), BDSSM_ERR_NULL);
    bdssm_decode_graph_destroy(NULL);
    bdssm_launch_override o = {3, 0, 0, 0};
    EXPECT(bdssm_set_launch_override(&o), BDSSM_ERR_UNSUPPORTED);
    EXPECT(bdssm_set_launch_override(NULL), BDSSM_OK);
    puts("host library sanitizer run: ok");
    return 0;
}
