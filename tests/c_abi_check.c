/*
 * A plain C11 client of include/art.h, built with gcc against libart.so by
 * tests/test_abi.py.  It makes host-only calls (no device is touched): the
 * ABI version, descriptor validation and workspace sizing, status strings,
 * and the error paths of art_decode_attention that are rejected before
 * anything is enqueued.  Prints "ok" and returns 0 when every check holds.
 */
#include <stdio.h>
#include <string.h>

#include "art.h"

static int failures = 0;
#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

int main(void) {
    CHECK(art_abi_version() == ART_ABI_VERSION);

    art_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 2;
    d.num_q_heads = 8;
    d.num_kv_heads = 2;
    d.head_dim = 128;
    d.q_dtype = ART_BF16;
    d.kv_dtype = ART_BF16;
    d.block_size = 16;
    d.max_blocks_per_seq = 8;
    d.num_blocks = 16;
    d.patience = 1;

    const size_t need = art_workspace_bytes(&d, 64);
    CHECK(need > 0);
    d.workspace = (void*)(uintptr_t)(1u << 20); /* any 256-byte aligned address: never dereferenced */
    d.workspace_bytes = need;
    CHECK(art_validate(&d, 64, 1e-3f, 1e-4f) == ART_OK);
    CHECK(art_validate(&d, 48, 1e-3f, 1e-4f) == ART_E_TILE);
    CHECK(art_validate(&d, 64, -1.f, 1e-4f) == ART_E_PARAM);
    CHECK(strlen(art_last_error()) > 0);

    d.kv_dtype = ART_I4; /* scales are required */
    CHECK(art_validate(&d, 64, 1e-3f, 1e-4f) == ART_E_NULL);
    d.kv_dtype = ART_BF16;

    d.tile_order = ART_ORDER_LIST; /* a caller's list needs tile_perm */
    CHECK(art_validate(&d, 64, 1e-3f, 1e-4f) == ART_E_NULL);
    d.tile_order = ART_ORDER_RECENT;
    CHECK(art_validate(&d, 64, 1e-3f, 1e-4f) == ART_OK);

    d.per_head_tables = 1;
    CHECK(art_workspace_bytes(&d, 64) > 0);
    d.per_head_tables = 0;

    /* rejected before anything is enqueued: missing required pointers */
    float out[1];
    int32_t used[1];
    CHECK(art_decode_attention(&d, NULL, NULL, NULL, NULL, NULL, 64, 1e-3f, 1e-4f, out, used, NULL) ==
          ART_E_NULL);
    CHECK(art_decode_attention(NULL, NULL, NULL, NULL, NULL, NULL, 64, 1e-3f, 1e-4f, out, used, NULL) ==
          ART_E_NULL);

    CHECK(strcmp(art_status_string(ART_OK), "ok") == 0);
    CHECK(art_status_string(ART_E_HIP) != NULL);

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
