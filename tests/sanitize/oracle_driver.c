/* The oracle over small random inputs of every storage format, layout, order,
 * per-head tables and the V skip, run under the sanitizers.  Prints "ok". */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int art_oracle_decode(int B, int Hq, int Hkv, int d, int q_dtype, int kv_dtype, int block_size,
                      int max_blocks_per_seq, int max_ctx, int num_blocks, const void* q, const void* k,
                      const void* v, const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                      const int32_t* ctx_lens, int tile, double eps_scale, double eps_dir, int patience,
                      double v_skip_eps, double* out, int32_t* tiles_used, double* trace, int trace_tiles,
                      int nthreads, int order, const int32_t* perm, int perm_stride, int per_head);

static uint32_t rs = 12345u;
static uint32_t rnd(void) { rs = rs * 1664525u + 1013904223u; return rs >> 8; }

int main(void) {
    enum { B = 2, Hkv = 2, Hq = 4, D = 16, BS = 16, MB = 6, NB = 16, CAP = MB * BS };
    const int tile = 16, nt_max = CAP / tile;
    float* qf = malloc(sizeof(float) * B * Hq * D);
    uint16_t* q16 = malloc(2 * B * Hq * D);
    const size_t rows = (size_t)NB * Hkv * BS > (size_t)B * Hkv * CAP ? (size_t)NB * Hkv * BS : (size_t)B * Hkv * CAP;
    float* kf = malloc(sizeof(float) * rows * D);
    float* vf = malloc(sizeof(float) * rows * D);
    uint16_t* k16 = malloc(2 * rows * D);
    uint16_t* v16 = malloc(2 * rows * D);
    int8_t* k8 = malloc(rows * D);
    int8_t* v8 = malloc(rows * D);
    uint8_t* k4 = malloc(rows * D / 2);
    uint8_t* v4 = malloc(rows * D / 2);
    uint16_t* ks = malloc(2 * rows);
    uint16_t* vs = malloc(2 * rows);
    for (size_t i = 0; i < (size_t)B * Hq * D; ++i) { qf[i] = (float)(rnd() % 200) / 100.f - 1.f; q16[i] = (uint16_t)(0x3c00 + rnd() % 0x200); }
    for (size_t i = 0; i < rows * D; ++i) {
        kf[i] = (float)(rnd() % 200) / 100.f - 1.f; vf[i] = (float)(rnd() % 200) / 100.f - 1.f;
        k16[i] = (uint16_t)(0x3c00 + rnd() % 0x200); v16[i] = (uint16_t)(0xbc00 + rnd() % 0x200);
        k8[i] = (int8_t)(rnd() % 255 - 127); v8[i] = (int8_t)(rnd() % 255 - 127);
    }
    for (size_t i = 0; i < rows * D / 2; ++i) { k4[i] = (uint8_t)rnd(); v4[i] = (uint8_t)rnd(); }
    for (size_t i = 0; i < rows; ++i) { ks[i] = (uint16_t)(0x1c00 + rnd() % 0x300); vs[i] = (uint16_t)(rnd() % 0x400); }
    int32_t table[B * Hkv * MB], lens[B * Hkv], perm[B * Hkv * 8];
    for (int i = 0; i < B * Hkv * MB; ++i) table[i] = (int32_t)(rnd() % NB);
    double* out = malloc(sizeof(double) * B * Hq * D);
    int32_t used[B * Hq];
    double* trace = malloc(sizeof(double) * B * Hq * nt_max * 8);
    int runs = 0;
    for (int kv = 0; kv < 4; ++kv)
        for (int paged = 0; paged < 2; ++paged)
            for (int order = 0; order < 3; ++order)
                for (int per_head = 0; per_head < 2; ++per_head)
                    for (int skip = 0; skip < 2; ++skip) {
                        const int nseq = per_head ? B * Hkv : B;
                        for (int sq = 0; sq < nseq; ++sq) lens[sq] = (int32_t)(rnd() % (CAP + 1));
                        for (int sq = 0; sq < nseq; ++sq) {
                            const int nt = (lens[sq] + tile - 1) / tile;
                            perm[sq * 8] = 0;
                            for (int t = 1; t < nt; ++t) perm[sq * 8 + t] = nt - t;
                        }
                        const void *k = kv == 0 ? (void*)kf : kv == 1 ? (void*)k16 : kv == 2 ? (void*)k8 : (void*)k4;
                        const void *v = kv == 0 ? (void*)vf : kv == 1 ? (void*)v16 : kv == 2 ? (void*)v8 : (void*)v4;
                        const int rc = art_oracle_decode(
                            B, Hq, Hkv, D, kv == 0 ? 0 : 1, kv, paged ? BS : 0, paged ? MB : 0, paged ? 0 : CAP,
                            paged ? NB : 0, kv == 0 ? (void*)qf : (void*)q16, k, v, kv >= 2 ? ks : NULL,
                            kv >= 2 ? vs : NULL, paged ? table : NULL, lens, tile, 1e-2, 1e-3, 1 + order, skip ? 1e-3 : 0.0,
                            out, used, trace, nt_max, 3, order, perm, 8, per_head);
                        if (rc != 0) { fprintf(stderr, "oracle returned %d\n", rc); return 1; }
                        ++runs;
                    }
    printf("ok %d\n", runs);
    free(qf); free(q16); free(kf); free(vf); free(k16); free(v16); free(k8); free(v8); free(k4); free(v4);
    free(ks); free(vs); free(out); free(trace);
    return 0;
}
