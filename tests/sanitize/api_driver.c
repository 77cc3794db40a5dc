/* Calls of the C ABI over many shapes, run under the sanitizers with the
 * launch stand-ins of api_stubs.cpp: validation, workspace sizing and the
 * host-side setup of art_decode_attention (device pointers are fake and
 * never dereferenced).  Prints "ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "art.h"

int main(void) {
    static const int32_t dtypes[] = {ART_F32, ART_BF16, ART_I8, ART_I4};
    static const int32_t tiles[] = {16, 32, 64, 128, 48};
    int calls = 0;
    for (int kvi = 0; kvi < 4; ++kvi)
        for (int hq = 1; hq <= 16; hq *= 2)
            for (int paged = 0; paged < 2; ++paged)
                for (int order = 0; order < 3; ++order)
                    for (int per_head = 0; per_head < 2; ++per_head)
                        for (int ti = 0; ti < 5; ++ti)
                            for (int art = 0; art < 3; ++art) {  /* full, ART + V skip, ART */
                                art_desc d;
                                memset(&d, 0, sizeof d);
                                d.batch = 3;
                                d.num_q_heads = hq * 2;
                                d.num_kv_heads = 2;
                                d.head_dim = (hq & 1) ? 64 : 128;
                                d.q_dtype = kvi == 0 ? ART_F32 : ART_BF16;
                                d.kv_dtype = dtypes[kvi];
                                d.block_size = paged ? 16 : 0;
                                d.max_blocks_per_seq = paged ? 9 : 0;
                                d.num_blocks = paged ? 40 : 0;
                                d.max_ctx = paged ? 0 : 144;
                                d.patience = 1 + order;
                                d.v_skip_eps = art == 1 ? 1e-6f : 0.f;
                                d.k_scale = d.v_scale = (kvi >= 2) ? (const void*)(uintptr_t)0x1000 : NULL;
                                d.tile_order = order;
                                d.tile_perm_stride = 16;
                                d.tile_perm = order == 2 ? (const int32_t*)(uintptr_t)0x2000 : NULL;
                                d.per_head_tables = per_head;
                                d.engine = (ti + order + art) % 7;  /* every engine, the round engine too */
                                const int tile = tiles[ti];
                                const size_t need = art_workspace_bytes(&d, tile);
                                d.workspace = (void*)(uintptr_t)(1u << 20);
                                d.workspace_bytes = need;
                                const float e = art ? 1e-3f : 0.f;
                                const int32_t rc = art_decode_attention(
                                    &d, (const void*)(uintptr_t)0x3000, (const void*)(uintptr_t)0x4000,
                                    (const void*)(uintptr_t)0x5000,
                                    paged ? (const int32_t*)(uintptr_t)0x6000 : NULL, (const int32_t*)(uintptr_t)0x7000,
                                    tile, e, e, (float*)(uintptr_t)0x8000, (int32_t*)(uintptr_t)0x9000, NULL);
                                if (need == 0 && rc == ART_OK) {
                                    fprintf(stderr, "an invalid desc was accepted\n");
                                    return 1;
                                }
                                (void)art_status_string(rc);
                                (void)art_last_error();
                                ++calls;
                            }
    printf("ok %d\n", calls);
    return 0;
}
