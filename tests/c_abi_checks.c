/* Host-side refusals of the C ABI, driven from plain C without a GPU.
 *
 * Every call below must fail one of the documented argument checks before any
 * HIP call, so the pointers are fake, far-apart, 16-byte-aligned addresses that
 * are never dereferenced.  tests/test_sanitizers.py builds this program against
 * a copy of the library whose host code (api.cpp) carries AddressSanitizer and
 * UndefinedBehaviorSanitizer, so an out-of-bounds access, overflow or other
 * undefined behaviour in the checks aborts the run.  It also round-trips the
 * tuning cache through a file (argv[1]) and reads the cache file argv[2], which
 * does not exist.  Exit status 0 = every check returned its documented status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bsattn.h"

static int failures = 0;

#define EXPECT(call, want)                                                                   \
    do {                                                                                     \
        const int got_ = (call);                                                             \
        if (got_ != (want)) {                                                                \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
                    (int)(want));                                                            \
            ++failures;                                                                      \
        }                                                                                    \
    } while (0)

#define A ((uintptr_t)1 << 20)
#define P(x) ((void*)(uintptr_t)(x))

int main(int argc, char** argv) {
    if (argc < 3) {
        fprintf(stderr, "usage: %s <cache file to write> <missing file>\n", argv[0]);
        return 2;
    }
    size_t n = 0;
    int cnt = 0;
    bsattn_tile_config cfg = {0, 0, 0, 0};
    const float nan_ = nanf("");

    /* status strings exist for every status, and for an unknown one */
    for (int s = BSATTN_OK; s <= BSATTN_ERR_IO; ++s)
        if (!bsattn_status_string(s) || strncmp(bsattn_status_string(s), "BSATTN", 6) != 0) ++failures;
    if (!bsattn_status_string(1234)) ++failures;

    /* sizes */
    EXPECT(bsattn_workspace_size(1, 1, 100, 64, 64, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_workspace_size(0, 1, 128, 64, 64, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_workspace_size(1, 1, 128, 64, 64, NULL), BSATTN_ERR_NULL);
    EXPECT(bsattn_workspace_size(1, 1, 128, 64, 64, &n), BSATTN_OK);
    EXPECT(bsattn_compact_workspace_size(1, 1, 1 << 16, 1 << 16, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_compact_workspace_size(1 << 30, 1 << 30, 4, 4, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_fp8_workspace_size(1, 1, 250, 64, 64, 64, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_bwd_workspace_size(1, 1, 250, 64, 64, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_ragged_dot_workspace_size(-1, 4, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_list_configs(7, 64, 64, 64, NULL, 0, &cnt), BSATTN_ERR_UNSUPPORTED);
    EXPECT(bsattn_list_configs(BSATTN_BF16, 128, 128, 128, NULL, 0, NULL), BSATTN_ERR_NULL);
    /* extreme sizes: every size computation must refuse them without overflowing */
    const int big = 2147483647, big128 = 2147483520; /* INT_MAX, the largest multiple of 128 */
    EXPECT(bsattn_workspace_size(big, big, big128, 128, 128, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_workspace_size(1, 1, big128, 64, 64, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_compact_workspace_size(big, big, big, big, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_fp8_workspace_size(big, big, big128, 128, 128, 128, &n), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_bwd_workspace_size(big, big, big128, 128, 128, &n), BSATTN_ERR_SHAPE);
    {
        const int rc_ = bsattn_ragged_dot_workspace_size(big, big, &n);
        if (rc_ == BSATTN_OK) ++failures;
    }

    /* forward: NULL, shape, dtype/D/block, alignment, scale, aliasing, workspace, config */
    const void *q = P(A), *k = P(3 * A), *v = P(5 * A);
    const uint8_t* mask = (const uint8_t*)P(7 * A);
    void* out = P(9 * A);
    float* lse = (float*)P(11 * A);
    void* ws = P(13 * A);
    const size_t wsb = 1 << 20;
#define FWD(q_, k_, v_, m_, o_, l_, B_, H_, S_, D_, bq_, bk_, sc_, dt_, ws_, wsb_, cfg_) \
    bsattn_fwd_config(q_, k_, v_, m_, o_, l_, B_, H_, S_, D_, bq_, bk_, sc_, dt_, ws_, wsb_, cfg_, NULL)
    EXPECT(FWD(NULL, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_NULL);
    EXPECT(FWD(q, k, v, NULL, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_NULL);
    EXPECT(FWD(q, k, v, mask, out, NULL, 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_NULL);
    EXPECT(FWD(q, k, v, mask, out, lse, 0, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_SHAPE);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, -1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_SHAPE);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 250, 64, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_SHAPE);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 1 << 22, 128, 128, 128, 0.1f, 1, ws, wsb, NULL), BSATTN_ERR_SHAPE);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 96, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_UNSUPPORTED);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 5, ws, wsb, NULL), BSATTN_ERR_UNSUPPORTED);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 32, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_UNSUPPORTED);
    EXPECT(FWD(P(A + 8), k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_ALIGN);
    EXPECT(FWD(q, k, v, mask, out, (float*)P(11 * A + 2), 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL),
           BSATTN_ERR_ALIGN);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, nan_, 1, ws, wsb, NULL), BSATTN_ERR_SCALE);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, INFINITY, 1, ws, wsb, NULL), BSATTN_ERR_SCALE);
    EXPECT(FWD(q, k, v, mask, P(A + 1024), lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL), BSATTN_ERR_ALIAS);
    EXPECT(FWD(q, k, v, mask, out, (float*)P(9 * A), 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, NULL),
           BSATTN_ERR_ALIAS);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, NULL, wsb, NULL), BSATTN_ERR_WORKSPACE);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, 16, NULL), BSATTN_ERR_WORKSPACE);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, P(3 * A), wsb, NULL), BSATTN_ERR_ALIAS);
    cfg = (bsattn_tile_config){256, 64, 8, 2}; /* row pairs need block_q 128 */
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, &cfg), BSATTN_ERR_UNSUPPORTED);
    cfg = (bsattn_tile_config){64, 48, 2, 1};
    EXPECT(FWD(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.125f, 1, ws, wsb, &cfg), BSATTN_ERR_UNSUPPORTED);
    EXPECT(bsattn_fwd(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, nan_, 1, ws, wsb, NULL), BSATTN_ERR_SCALE);
    EXPECT(FWD(q, k, v, mask, out, lse, big, big, big128, 128, 128, 128, 0.1f, 1, ws, wsb, NULL), BSATTN_ERR_SHAPE);
    EXPECT(FWD(q, k, v, mask, out, lse, 1, big, 1 << 20, 128, 128, 128, 0.1f, 1, ws, wsb, NULL), BSATTN_ERR_SHAPE);

    /* plan, planned, compacted, compaction, no-allocation forward */
    EXPECT(bsattn_plan(NULL, 1, 2, 512, 128, 64, ws, wsb, NULL), BSATTN_ERR_NULL);
    EXPECT(bsattn_plan(mask, 1, 2, 500, 128, 64, ws, wsb, NULL), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_plan(mask, 1, 2, 512, 32, 64, ws, wsb, NULL), BSATTN_ERR_UNSUPPORTED);
    EXPECT(bsattn_plan(mask, 1, 2, 512, 128, 64, ws, 64, NULL), BSATTN_ERR_WORKSPACE);
    EXPECT(bsattn_plan(mask, 1, 2, 512, 128, 64, P(13 * A + 2), wsb, NULL), BSATTN_ERR_ALIGN);
    EXPECT(bsattn_fwd_planned(q, k, v, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, NULL, wsb, NULL, NULL),
           BSATTN_ERR_NULL);
    EXPECT(bsattn_fwd_planned(q, k, v, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, ws, 16, NULL, NULL),
           BSATTN_ERR_WORKSPACE);
    EXPECT(bsattn_fwd_planned(q, k, v, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, P(9 * A + 512), wsb, NULL, NULL),
           BSATTN_ERR_ALIAS);
    EXPECT(bsattn_fwd_compacted(q, k, v, NULL, (const int32_t*)P(8 * A), 16, out, lse, 1, 1, 256, 64, 64, 64,
                                0.1f, 1, NULL, NULL),
           BSATTN_ERR_NULL);
    EXPECT(bsattn_fwd_compacted(q, k, v, (const int32_t*)P(7 * A + 2), (const int32_t*)P(8 * A), 16, out, lse, 1,
                                1, 256, 64, 64, 64, 0.1f, 1, NULL, NULL),
           BSATTN_ERR_ALIGN);
    EXPECT(bsattn_compact_mask(NULL, 1, 1, 4, 4, (int32_t*)P(A), (int32_t*)P(2 * A), P(3 * A), wsb, NULL),
           BSATTN_ERR_NULL);
    EXPECT(bsattn_compact_mask(mask, 1, 1, 4, 4, (int32_t*)P(A), (int32_t*)P(2 * A), P(3 * A), 8, NULL),
           BSATTN_ERR_WORKSPACE);
    EXPECT(bsattn_fwd_noalloc(q, k, v, NULL, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, NULL, NULL),
           BSATTN_ERR_NULL);
    EXPECT(bsattn_fwd_noalloc(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, nan_, 1, NULL, NULL),
           BSATTN_ERR_SCALE);
    EXPECT(bsattn_fwd_noalloc(P(1ull << 40), P(2ull << 40), P(3ull << 40), mask, P(4ull << 40),
                              (float*)P(5ull << 40), 1, 64, 65536, 64, 128, 128, 0.1f, 1, NULL, NULL),
           BSATTN_ERR_WORKSPACE);
    if (bsattn_noalloc_max_bytes() != ((size_t)16 << 20)) ++failures;

    /* element-level masks */
    const uint8_t* st = (const uint8_t*)P(7 * A);
    const int32_t* pidx = (const int32_t*)P(8 * A);
    const uint32_t* pbits = (const uint32_t*)P(15 * A);
    EXPECT(bsattn_fwd_elem(q, k, v, NULL, pidx, pbits, 2, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, ws, wsb,
                           NULL, NULL),
           BSATTN_ERR_NULL);
    EXPECT(bsattn_fwd_elem(q, k, v, st, pidx, pbits, 0, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, ws, wsb,
                           NULL, NULL),
           BSATTN_ERR_SHAPE);
    EXPECT(bsattn_fwd_elem(q, k, v, st, pidx, pbits, 40000, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, ws, wsb,
                           NULL, NULL),
           BSATTN_ERR_SHAPE);
    EXPECT(bsattn_fwd_elem(q, k, v, st, (const int32_t*)P(8 * A + 2), pbits, 2, out, lse, 1, 1, 256, 64, 64, 64,
                           0.1f, 1, ws, wsb, NULL, NULL),
           BSATTN_ERR_ALIGN);
    EXPECT(bsattn_plan_elem(st, pidx, 2, 1, 1, 256, 64, 64, ws, 8, NULL), BSATTN_ERR_WORKSPACE);
    EXPECT(bsattn_list_configs_elem(7, 64, 64, 64, NULL, 0, &cnt), BSATTN_ERR_UNSUPPORTED);

    /* fp8 */
    EXPECT(bsattn_fwd_fp8(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, nan_, ws, 1 << 22, NULL),
           BSATTN_ERR_SCALE);
    EXPECT(bsattn_fwd_fp8(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, ws, 16, NULL),
           BSATTN_ERR_WORKSPACE);
    EXPECT(bsattn_fwd_fp8(q, k, v, NULL, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, ws, 1 << 22, NULL),
           BSATTN_ERR_NULL);

    /* backward */
    void *dq = P(17 * A), *dk = P(19 * A), *dv = P(21 * A);
    const void* dout = P(23 * A);
    EXPECT(bsattn_bwd(q, k, v, out, lse, NULL, mask, 1, 1, 256, 64, 64, 64, 0.1f, 1, dq, dk, dv, 1, ws, 1 << 24,
                      NULL),
           BSATTN_ERR_NULL);
    EXPECT(bsattn_bwd(q, k, v, out, lse, dout, mask, 1, 1, 256, 96, 64, 64, 0.1f, 1, dq, dk, dv, 1, ws, 1 << 24,
                      NULL),
           BSATTN_ERR_UNSUPPORTED);
    EXPECT(bsattn_bwd(q, k, v, out, lse, dout, mask, 1, 1, 256, 64, 64, 64, 0.1f, 1, dq, dk, dv, 1, ws, 16, NULL),
           BSATTN_ERR_WORKSPACE);
    EXPECT(bsattn_bwd(q, k, v, out, lse, dout, mask, 1, 1, 256, 64, 64, 64, 0.1f, 1, P(A + 64), dk, dv, 1, ws,
                      1 << 24, NULL),
           BSATTN_ERR_ALIAS);
    EXPECT(bsattn_bwd_planned(q, k, v, out, lse, dout, 1, 1, 256, 64, 64, 64, 0.1f, 1, dq, dk, dv, 1, 0, ws,
                              1 << 24, NULL),
           BSATTN_ERR_UNSUPPORTED);

    /* ragged dot */
    const void *lhs = P(A), *rhs = P(3 * A);
    const int32_t* gs = (const int32_t*)P(5 * A);
    void* rout = P(7 * A);
    EXPECT(bsattn_ragged_dot(lhs, rhs, NULL, rout, 256, 64, 128, 2, 1, 1, ws, wsb, NULL), BSATTN_ERR_NULL);
    EXPECT(bsattn_ragged_dot(lhs, rhs, gs, rout, 256, 60, 128, 2, 1, 1, ws, wsb, NULL), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_ragged_dot(lhs, rhs, gs, rout, 256, 64, 100, 2, 1, 1, ws, wsb, NULL), BSATTN_ERR_SHAPE);
    EXPECT(bsattn_ragged_dot(lhs, rhs, gs, rout, 256, 64, 128, 2, 0, 1, ws, wsb, NULL), BSATTN_ERR_UNSUPPORTED);
    EXPECT(bsattn_ragged_dot(lhs, rhs, gs, P(A + 16), 256, 64, 128, 2, 1, 1, ws, wsb, NULL), BSATTN_ERR_ALIAS);
    EXPECT(bsattn_ragged_dot(lhs, rhs, gs, rout, 256, 64, 128, 2, 1, 1, ws, 4, NULL), BSATTN_ERR_WORKSPACE);
    {
        const int rc_ = bsattn_ragged_dot(lhs, rhs, gs, rout, big, 1 << 30, 1 << 30, big, 1, 1, ws, wsb, NULL);
        if (rc_ == BSATTN_OK || rc_ == BSATTN_ERR_HIP) ++failures;
    }
    EXPECT(bsattn_bwd(q, k, v, out, lse, dout, mask, big, big, big128, 128, 128, 128, 0.1f, 1, dq, dk, dv, 1, ws,
                      1 << 24, NULL),
           BSATTN_ERR_SHAPE);
    EXPECT(bsattn_fwd_elem(q, k, v, st, pidx, pbits, 2, out, lse, big, big, big128, 128, 128, 128, 0.1f, 1, ws,
                           wsb, NULL, NULL),
           BSATTN_ERR_SHAPE);
    EXPECT(bsattn_fwd_fp8(q, k, v, mask, out, lse, big, big, big128, 128, 128, 128, 0.1f, ws, 1 << 22, NULL),
           BSATTN_ERR_SHAPE);

    /* autotuner arguments and the tuning cache (host only) */
    bsattn_tile_config best;
    int nres = 0;
    EXPECT(bsattn_autotune(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, ws, wsb, 1, 1, NULL, NULL, 0,
                           &nres, NULL, NULL),
           BSATTN_ERR_NULL);
    EXPECT(bsattn_autotune(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, ws, wsb, 1, 0, &best, NULL, 0,
                           &nres, NULL, NULL),
           BSATTN_ERR_SHAPE);
    EXPECT(bsattn_autotune(q, k, v, mask, out, lse, 1, 1, 256, 64, 64, 64, 0.1f, 1, ws, 4, 1, 1, &best, NULL, 0,
                           &nres, NULL, NULL),
           BSATTN_ERR_WORKSPACE);
    EXPECT(bsattn_tune_lookup(1, 128, 4, 16, 2048, 128, 128, 16384, NULL), BSATTN_ERR_NULL);
    EXPECT(bsattn_tune_lookup(1, 128, 4, 16, 2000, 128, 128, 16384, &cfg), BSATTN_ERR_SHAPE);
    bsattn_clear_tune_cache();
    EXPECT(bsattn_tune_lookup(1, 128, 4, 16, 2048, 128, 128, 16384, &cfg), BSATTN_ERR_UNSUPPORTED);
    FILE* f = fopen(argv[1], "w");
    if (!f) return 3;
    fprintf(f, "{\"bsattn_tune_cache\": 1, \"entries\": [\n"
               "  {\"dtype\": 1, \"D\": 128, \"block_q\": 128, \"block_k\": 128, \"S\": 2048, \"BH\": 64, "
               "\"mask_bucket\": 4, \"tile_q\": 128, \"tile_k\": 64, \"waves\": 4, \"stages\": 2, "
               "\"t_mean_s\": 1.0e-04},\n"
               "  {\"dtype\": 1, \"D\": 128, \"block_q\": 128, \"block_k\": 128, \"S\": 2048, \"BH\": 64, "
               "\"mask_bucket\": 8, \"tile_q\": 256, \"tile_k\": 128, \"waves\": 8, \"stages\": 2, "
               "\"t_mean_s\": 1.0e-04}\n]}\n");
    fclose(f);
    EXPECT(bsattn_load_tune_cache(argv[1]), BSATTN_OK);
    EXPECT(bsattn_load_tune_cache(argv[2]), BSATTN_ERR_IO);
    EXPECT(bsattn_load_tune_cache(NULL), BSATTN_ERR_NULL);
    EXPECT(bsattn_tune_lookup(1, 128, 4, 16, 2048, 128, 128, 4096, &cfg), BSATTN_OK);
    if (cfg.tile_q != 128 || cfg.tile_k != 64) ++failures;
    EXPECT(bsattn_tune_lookup(1, 128, 4, 16, 2048, 128, 128, -1, &cfg), BSATTN_OK);
    if (cfg.tile_q != 256 || cfg.tile_k != 128) ++failures;
    bsattn_clear_tune_cache();

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("all host checks returned their documented status\n");
    return 0;
}
