/* A C99 program against include/sva.h: the library's host-only calls used
 * from plain C, with no device.  tests/test_abi.py builds it with gcc
 * (-std=c99 -pedantic -Werror), links libsva.so and runs it; it prints "ok"
 * and exits 0 when every check holds.
 *
 * Shape: 1,024 video tokens on a 4 x 16 x 16 latent grid, 2 heads, head
 * width 64, 64-token blocks, sparsity 0.5.  With the default 4 x 4 x 4
 * tiles every tile is one block, so the tile order and the budget can be
 * written out by hand. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sva.h"

#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
            return 1;                                                         \
        }                                                                     \
    } while (0)

static int tile_position(int t, int h, int w) {
    /* tiles of 4 x 4 x 4 in (t, h, w) order, 4 x 4 tiles per frame group;
     * tokens inside a tile in (t, h, w) order */
    const int tile = ((t / 4) * 4 + h / 4) * 4 + w / 4;
    return tile * 64 + ((t % 4) * 4 + h % 4) * 4 + w % 4;
}

int main(void) {
    sva_plan_desc desc;
    sva_plan_info info;
    int32_t perm[1024];
    int32_t row_ptr[17];
    uint8_t forced[16 * 16];
    int t, h, w, i;

    CHECK(sva_plan_desc_init(&desc, 1, 2, 4, 16, 16, 64, 64, 0.5, 0u) == SVA_OK);
    CHECK(sva_plan_query(&desc, &info) == SVA_OK);
    CHECK(info.n_video == 1024 && info.N == 1024 && info.Np == 1024);
    CHECK(info.nB == 16 && info.nB_video == 16 && info.k == 8 && info.dense == 0);
    CHECK(info.nnz_per_head == 16 * 8 && info.nnz == 2 * 16 * 8);
    CHECK(info.tile[0] == 4 && info.tile[1] == 4 && info.tile[2] == 4);
    CHECK(info.rope_split[0] == 16 && info.rope_split[1] == 24 && info.rope_split[2] == 24);
    CHECK(info.select_workspace_bytes > 0);

    CHECK(sva_plan_host_tables(&desc, perm, row_ptr, forced) == SVA_OK);
    for (t = 0; t < 4; ++t)
        for (h = 0; h < 16; ++h)
            for (w = 0; w < 16; ++w)
                CHECK(perm[(t * 16 + h) * 16 + w] == tile_position(t, h, w));
    for (i = 0; i <= 16; ++i) CHECK(row_ptr[i] == i * 8);
    for (i = 0; i < 16 * 16; ++i) CHECK(forced[i] == 0);
    /* NULL skips a table */
    CHECK(sva_plan_host_tables(&desc, NULL, row_ptr, NULL) == SVA_OK);

    /* a dense plan keeps every block */
    CHECK(sva_plan_desc_init(&desc, 1, 2, 4, 16, 16, 64, 64, 0.5, SVA_DENSE) == SVA_OK);
    CHECK(sva_plan_query(&desc, &info) == SVA_OK);
    CHECK(info.dense == 1 && info.k == 16 && info.nnz_per_head == 16 * 16);

    /* errors come back as status codes with a message */
    CHECK(sva_plan_desc_init(&desc, 1, 2, 4, 16, 16, 96, 64, 0.5, 0u) == SVA_OK);
    CHECK(sva_plan_query(&desc, &info) == SVA_ERR_UNSUPPORTED);
    CHECK(strlen(sva_last_error()) > 0);
    CHECK(sva_plan_desc_init(&desc, 1, 2, 4, 16, 16, 64, 64, 1.5, 0u) == SVA_OK);
    CHECK(sva_plan_query(&desc, &info) == SVA_ERR_INVALID_ARG);
    CHECK(sva_plan_query(NULL, &info) == SVA_ERR_INVALID_ARG);
    CHECK(sva_plan_desc_init(NULL, 1, 2, 4, 16, 16, 64, 64, 0.5, 0u) == SVA_ERR_INVALID_ARG);
    CHECK(strcmp(sva_status_string(SVA_OK), "ok") == 0);
    CHECK(strcmp(sva_status_string(SVA_ERR_WORKSPACE), "workspace too small") == 0);

    printf("ok\n");
    return 0;
}
