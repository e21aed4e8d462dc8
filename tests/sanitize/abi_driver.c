/*
 * Runs the host-side code of the C ABI (include/dspark.h) that needs no GPU:
 * the workspace-size functions over a grid of sizes (including the limits and
 * sizes past them), the argument checks of every entry point (each call below
 * fails a check, or has nothing to do, before any HIP call), the status
 * strings and the wait-limit setting. Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code of the library, so an overflow
 * in a size computation, a bad pointer or undefined arithmetic aborts it.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dspark.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

int main(void) {
    const int Bs[] = {-1, 0, 1, 3, 4, 5, 96, 128, 129, 4096, 65535, 65536};
    const int Ks[] = {-1, 0, 1, 7, 16, 255, 256};
    const int Vs[] = {-8, 0, 4, 8, 4100, 4096, 200064, 262144, 262152, 1 << 24};
    const int rs[] = {-32, 0, 32, 48, 256, 1024, 2048};
    size_t nonzero = 0;
    for (size_t i = 0; i < sizeof Bs / sizeof *Bs; ++i)
        for (size_t j = 0; j < sizeof Ks / sizeof *Ks; ++j)
            for (size_t l = 0; l < sizeof Vs / sizeof *Vs; ++l) {
                for (size_t m = 0; m < sizeof rs / sizeof *rs; ++m) {
                    const size_t n = dspark_workspace_bytes(Bs[i], Ks[j], Vs[l], rs[m]);
                    nonzero += n != 0;
                    if (Bs[i] < 0 || Ks[j] < 0 || Vs[l] <= 0 || rs[m] <= 0 || Ks[j] > 255 || rs[m] > 1024 ||
                        Vs[l] % 8 || rs[m] % 32)
                        CHECK(n == 0);
                }
                (void)dspark_verify_workspace_bytes(Bs[i], Ks[j], Vs[l]);
                (void)dspark_verify_block_workspace_bytes(Bs[i], Ks[j], Vs[l]);
            }
    CHECK(nonzero > 0);
    const int Ls[] = {-1, 1, 8, 9100, 1 << 20};
    for (size_t i = 0; i < sizeof Bs / sizeof *Bs; ++i)
        for (size_t l = 0; l < sizeof Ls / sizeof *Ls; ++l)
            for (int K = 0; K <= 9; K += 3) {
                (void)dspark_window_attention_workspace_bytes(Bs[i], K, 64, 4, 128, Ls[l], 4096);
                (void)dspark_window_attention_workspace_bytes(Bs[i], K, 16, 1, 128, Ls[l], 64);
                (void)dspark_window_attention_workspace_bytes(Bs[i], K, 17, 1, 96, Ls[l], 0);
            }

    /* argument checks of the draft block: each fails before anything is enqueued */
    char buf[64] __attribute__((aligned(16)));
    void* P = buf;                      /* an aligned host address, never dereferenced */
    void* M = buf + 4;                  /* misaligned */
    const size_t ws = dspark_workspace_bytes(2, 7, 4096, 32);
    CHECK(dspark_draft_block(P, 0, P, P, P, P, P, P, NULL, 2, 7, 4100, 32, P, P, P, P, ws, NULL) == DSPARK_ERR_UNSUPPORTED);
    CHECK(dspark_draft_block(P, 0, P, P, P, P, P, P, NULL, 2, 7, 4096, 48, P, P, P, P, ws, NULL) == DSPARK_ERR_UNSUPPORTED);
    CHECK(dspark_draft_block(P, 0, P, P, P, P, P, P, NULL, -1, 7, 4096, 32, P, P, P, P, ws, NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_draft_block(P, 9, P, P, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, P, ws, NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_draft_block(NULL, 0, P, P, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, P, ws, NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_draft_block(M, 0, P, P, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, P, ws, NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_draft_block(P, 0, P, P, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, NULL, ws, NULL) == DSPARK_ERR_WORKSPACE);
    CHECK(dspark_draft_block(P, 0, P, P, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, P, 100, NULL) == DSPARK_ERR_WORKSPACE);
    CHECK(dspark_draft_block(NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 7, 4096, 32, NULL, NULL, NULL, NULL, 0,
                             NULL) == DSPARK_OK);
    CHECK(dspark_draft_block_chunked(P, 0, P, P, P, P, P, P, NULL, 2, 7, 4096, 32, 100, P, P, P, P, ws, NULL) ==
          DSPARK_ERR_UNSUPPORTED);
    CHECK(dspark_draft_block_events(P, 0, P, P, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, P, ws, NULL, NULL, 0) ==
          DSPARK_ERR_ARG);
    /* packed W: sizes no resident plan runs, bad arguments, the packed block's own checks */
    const int pVs[] = {-8, 0, 4, 4100, 262152, 1 << 24};
    const int prs[] = {-32, 0, 48, 288, 1024};
    for (size_t l = 0; l < sizeof pVs / sizeof *pVs; ++l)
        for (size_t m = 0; m < sizeof prs / sizeof *prs; ++m) {
            CHECK(dspark_packed_w_bytes(pVs[l], prs[m]) == 0);
            CHECK(dspark_pack_w(P, pVs[l], prs[m], P, 1 << 20, NULL) != DSPARK_OK);
        }
    CHECK(dspark_draft_block_packed(P, 0, P, P, NULL, 0, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, P, ws, NULL, NULL, 0) ==
          DSPARK_ERR_ARG);
    CHECK(dspark_draft_block_packed(P, 0, P, P, M, 1, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, P, ws, NULL, NULL, 0) ==
          DSPARK_ERR_ARG);
    CHECK(dspark_draft_block_packed(P, 0, P, P, P, 1, P, P, P, P, NULL, 2, 7, 4100, 32, P, P, P, P, ws, NULL, NULL, 0) ==
          DSPARK_ERR_UNSUPPORTED);
    CHECK(dspark_draft_block_packed(P, 0, P, P, P, 1, P, P, P, P, NULL, 2, 7, 4096, 32, P, P, P, NULL, ws, NULL, NULL, 0) ==
          DSPARK_ERR_WORKSPACE);
    /* the slot-indexed entry */
    CHECK(dspark_draft_block_slots(P, 0, P, P, NULL, 0, P, P, P, P, NULL, NULL, 4, 2, 7, 4096, 32, P, P, P, P, ws,
                                   NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_draft_block_slots(P, 0, P, P, NULL, 0, P, P, P, P, NULL, P, 0, 2, 7, 4096, 32, P, P, P, P, ws,
                                   NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_draft_block_slots(P, 0, P, P, NULL, 0, P, P, P, P, NULL, P, 4, 2, 7, 4100, 32, P, P, P, P, ws,
                                   NULL) == DSPARK_ERR_UNSUPPORTED);
    CHECK(dspark_draft_block_slots(P, 0, P, P, NULL, 0, P, P, P, P, NULL, P, 4, 2, 7, 4096, 32, P, P, M, P, ws,
                                   NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_draft_block_slots(P, 0, P, P, NULL, 0, P, P, P, P, NULL, P, 4, 2, 7, 4096, 32, P, P, P, NULL, ws,
                                   NULL) == DSPARK_ERR_WORKSPACE);
    CHECK(dspark_launch_plan(2, 7, 4100, 32, NULL, 0) == DSPARK_ERR_UNSUPPORTED);
    CHECK(dspark_launch_plan(0, 7, 4096, 32, NULL, 0) == 0);

    /* verification and attention argument checks */
    const size_t vws = dspark_verify_workspace_bytes(2, 3, 64);
    CHECK(dspark_verify_standard(P, P, P, P, P, 2, 3, 62, P, P, P, vws, NULL) == DSPARK_ERR_UNSUPPORTED);
    CHECK(dspark_verify_standard(P, M, P, P, P, 2, 3, 64, P, P, P, vws, NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_verify_standard(P, P, P, P, P, 2, 3, 64, P, P, NULL, vws, NULL) == DSPARK_ERR_WORKSPACE);
    CHECK(dspark_verify_standard(NULL, NULL, NULL, NULL, NULL, 0, 3, 64, NULL, NULL, NULL, 0, NULL) == DSPARK_OK);
    const size_t bws = dspark_verify_block_workspace_bytes(2, 3, 64);
    CHECK(dspark_verify_block(P, P, P, P, P, 2, 256, 64, P, P, P, bws, NULL) == DSPARK_ERR_UNSUPPORTED);
    CHECK(dspark_verify_block(P, P, NULL, P, P, 2, 3, 64, P, P, P, bws, NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_verify_block(P, P, P, P, P, 2, 3, 64, P, P, P, 8, NULL) == DSPARK_ERR_WORKSPACE);
    const size_t aws = dspark_window_attention_workspace_bytes(2, 7, 64, 4, 128, 9100, 4096);
    CHECK(dspark_window_block_attention(P, P, P, P, 2, 7, 64, 4, 96, 9100, 4096, 0.1f, P, P, P, aws, NULL) != DSPARK_OK);
    CHECK(dspark_window_block_attention(P, P, P, P, 2, 7, 64, 4, 128, 9100, 4096, -1.0f, P, P, P, aws, NULL) ==
          DSPARK_ERR_ARG);
    CHECK(dspark_window_block_attention(P, P, P, P, 2, 7, 64, 4, 128, 9100, 4096, 0.1f, P, P, P, 0, NULL) ==
          DSPARK_ERR_WORKSPACE);
    CHECK(dspark_window_block_attention_layout(P, P, P, P, 2, 7, 64, 4, 128, 9100, 4096, 0.1f, 2, P, P, P, aws,
                                               NULL) == DSPARK_ERR_ARG);
    CHECK(dspark_window_block_attention_layout(P, P, P, P, 2, 7, 64, 4, 128, 9100, 4096, 0.1f,
                                               DSPARK_KV_LAYOUT_BHLD, P, P, P, 0, NULL) == DSPARK_ERR_WORKSPACE);
    CHECK(dspark_window_block_attention_layout(NULL, NULL, NULL, NULL, 0, 7, 64, 4, 128, 9100, 4096, 0.1f,
                                               DSPARK_KV_LAYOUT_BHLD, NULL, NULL, NULL, 0, NULL) == DSPARK_OK);

    CHECK(dspark_block_status(NULL, NULL) == DSPARK_ERR_ARG);
    const unsigned prev = dspark_set_wait_limit(3);
    CHECK(dspark_set_wait_limit(prev) == 3);
    for (int s = -10; s <= 10; ++s) CHECK(dspark_status_string(s) != NULL && strlen(dspark_status_string(s)) > 0);
    if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
    printf("abi driver ok\n");
    return 0;
}
