/* A C caller of libssu: include/ssu.h compiled as C11, every entry point
 * called on inputs that need no GPU (validation errors and no-op sizes).
 * Prints "ok" and returns 0 when every call behaves as the header states. */
#include <stdio.h>
#include <string.h>

#include "ssu.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            printf("FAILED line %d: %s (%s)\n", __LINE__, #cond,        \
                   ssu_last_error());                                  \
            ++failures;                                                \
        }                                                              \
    } while (0)

int main(void)
{
    EXPECT(ssu_abi_version() == SSU_ABI_VERSION);
    EXPECT(strcmp(ssu_status_string(SSU_ERR_MISALIGNED), "SSU_ERR_MISALIGNED") == 0);

    /* handles */
    ssu_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.nheads = 16, cfg.headdim = 64, cfg.dstate = 128, cfg.ngroups = 1;
    cfg.dt_softplus = 1, cfg.tile = -1, cfg.device = -1;
    ssu_handle *h = NULL;
    EXPECT(ssu_create(&cfg, &h) == SSU_OK && h != NULL);
    ssu_config bad = cfg;
    bad.dstate = 100;
    ssu_handle *h2 = NULL;
    EXPECT(ssu_create(&bad, &h2) == SSU_ERR_UNSUPPORTED && h2 == NULL);
    bad = cfg;
    bad.ngroups = 3;
    EXPECT(ssu_create(&bad, &h2) == SSU_ERR_INVALID_ARGUMENT);
    EXPECT(ssu_create(NULL, &h2) == SSU_ERR_INVALID_ARGUMENT);

    /* tiles */
    EXPECT(ssu_tile_count() > 0);
    ssu_tile_desc d;
    EXPECT(ssu_tile_info(0, &d) == SSU_OK && d.dstate > 0 && d.name[0] != '\0');
    EXPECT(ssu_tile_info(ssu_tile_count(), &d) == SSU_ERR_INVALID_ARGUMENT);
    int32_t t = ssu_select_tile(h, 512);
    EXPECT(t >= 0 && ssu_tile_info(t, &d) == SSU_OK && d.dstate == 128);
    EXPECT(ssu_select_tile_tokens(h, 512, 3) >= 0);
    EXPECT(ssu_select_tile(NULL, 512) == -1);

    /* the decode step: batch 0 is a no-op; bad sizes are rejected */
    ssu_args a;
    memset(&a, 0, sizeof a);
    EXPECT(ssu_update(h, &a, NULL) == SSU_OK);
    EXPECT(ssu_check_indices(&a, NULL) == SSU_OK);
    a.batch = -1;
    EXPECT(ssu_update(h, &a, NULL) == SSU_ERR_INVALID_ARGUMENT);
    a.batch = 4; /* a null state view */
    EXPECT(ssu_update(h, &a, NULL) == SSU_ERR_INVALID_ARGUMENT);
    EXPECT(ssu_update(NULL, &a, NULL) == SSU_ERR_INVALID_ARGUMENT);

    ssu_tokens_args ta;
    memset(&ta, 0, sizeof ta);
    ta.ntokens = 3;
    EXPECT(ssu_update_tokens(h, &ta, NULL) == SSU_OK);
    ta.batch = 2, ta.ntokens = 0;
    EXPECT(ssu_update_tokens(h, &ta, NULL) == SSU_ERR_INVALID_ARGUMENT);

    /* block copies */
    EXPECT(ssu_copy_tile_count() > 0 && ssu_copy_tile_name(0)[0] != '\0');
    EXPECT(ssu_copy_tile_name(-1)[0] == '\0');
    ssu_block_tensor bt;
    memset(&bt, 0, sizeof bt);
    EXPECT(ssu_copy_blocks(&bt, 1, NULL, NULL, 0, -1, NULL) == SSU_OK);
    EXPECT(ssu_copy_blocks(&bt, -1, NULL, NULL, 1, -1, NULL) == SSU_ERR_INVALID_ARGUMENT);

    /* the scan */
    EXPECT(ssu_scan_tile_count() > 0 && ssu_scan_tile_name(0)[0] != '\0');
    EXPECT(ssu_scan_select_tile(NULL, 0) == -1);
    ssu_scan_args sa;
    memset(&sa, 0, sizeof sa);
    sa.dim = 1024, sa.dstate = 16, sa.ngroups = 1, sa.seqlen = 4096, sa.delta_softplus = 1;
    EXPECT(ssu_scan(&sa, 512, -1, NULL) == SSU_OK); /* batch 0 */
    sa.batch = 1, sa.dstate = 65;
    EXPECT(ssu_scan(&sa, 512, -1, NULL) == SSU_ERR_UNSUPPORTED);
    sa.dstate = 16;
    EXPECT(ssu_scan(&sa, 512, -1, NULL) == SSU_ERR_INVALID_ARGUMENT); /* null state */
    EXPECT(ssu_scan(NULL, 512, -1, NULL) == SSU_ERR_INVALID_ARGUMENT);

    ssu_destroy(h);
    ssu_destroy(NULL);
    if (failures)
        return 1;
    printf("ok\n");
    return 0;
}
