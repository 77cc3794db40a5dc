/*
 * Plain fp64 CPU oracle for ART-terminated decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source, header, table or helper
 * with the HIP library.
 *
 * What it computes (sources: the gist.science technical summary of
 * "ART: Runtime Attention Termination", arXiv 2606.00024, sections 2.1-2.4;
 * the puntofijo.es article on skipping V dequantisation in llama.cpp):
 *
 *   For every batch row b and query head h, one decode query attends over the
 *   first n = ctx_lens[b] cached positions of KV head g = h / (Hq/Hkv).  With
 *   per-head tables each (b, g) has its own length and block table: the
 *   positions a per-head retention or eviction policy kept, in order (ART
 *   summary, section 2.4: ART runs on top of such policies unchanged).  The
 *   positions are visited in tiles of T consecutive tokens (ART summary,
 *   section 2.1: tile-wise incremental attention that exposes the running
 *   output), tile 0 first and by default in ascending order; section 2.4
 *   lets the tile sequence be reordered (recency-first, importance-first:
 *   see visit_tile below).  After each tile the running softmax output
 *   O(t) = acc / l is formed and its first min(8, d) dimensions are the probe
 *   x(t) (section 2.2: a cheap probe vector of the partial output).
 *   From tile 1 on, two changes against the previous probe are measured
 *   (section 2.2, items 1 and 2):
 *       d_scale = | ||x(t)|| - ||x(t-1)|| | / ||x(t-1)||
 *       d_dir   = max(0, 1 - cos(x(t), x(t-1)))
 *   A tile passes when both are strictly below their thresholds (section
 *   2.2: both must fall below simultaneously).  After `patience` consecutive
 *   passing tiles (section 2.3) the traversal stops: tiles_used = t + 1 (t
 *   counts visiting steps) and the remaining tiles are never visited.  Tile
 *   0 is always evaluated before any stop (section 2.4, attention sinks):
 *   every order visits it first.  Without a stop, tiles_used = ceil(n / T).
 *
 *   Optional V skip (puntofijo.es: flash attention forms the softmax weights
 *   before touching V, so V rows whose weight is negligible need not be
 *   dequantised): with v_skip_eps > 0, position j of tile t is dropped from
 *   the V sum when exp(s_j - M_t) < v_skip_eps, M_t being the running
 *   maximum score through tile t.  Its weight still counts in l.
 *
 * Readings where the pages are silent are listed in the design notes; the
 * ones this file depends on: scores are q.k / sqrt(d); a probe of norm zero
 * makes both metrics +infinity (never passes); ctx_len 0 gives out = 0 and
 * tiles_used = 0; int8 values are dequantised as int8 * fp16 scale per
 * (token, KV head); int4 values likewise, as signed 4-bit codes stored two
 * per byte, element 2i in the low nibble of byte i (a format of this
 * library: the pages name lower-bit caches but do not specify a codec).
 *
 * Pins: see tests/test_oracle.py (brute-force softmax attention, prefix
 * identity, convexity, constant-V closed form, designed probe sequences,
 * paged-layout permutation, GQA replication, int8 dequant identity, V-skip
 * limits and error bound, output awareness, tile orders against physically
 * permuted caches and permutation invariance of full attention).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ODT_F32 = 0, ODT_BF16 = 1, ODT_I8 = 2, ODT_I4 = 3 };

/* trace record per (b, h, tile): see ORACLE_TRACE_FIELDS in oracle/__init__.py */
#define TRACE_FIELDS 8
/* 0 m (running max after the tile), 1 l, 2 d_scale, 3 d_dir, 4 streak,
   5 V rows kept in the tile, 6 ||x(t)||, 7 1 if the tile was evaluated */

typedef struct {
    int B, Hq, Hkv, d, q_dtype, kv_dtype;
    int block_size, max_blocks_per_seq, max_ctx, num_blocks;
    const void *q, *k, *v;
    const uint16_t *k_scale, *v_scale;
    const int32_t *block_table, *ctx_lens;
    int tile, patience;
    double eps_scale, eps_dir, v_skip_eps;
    double *out;
    int32_t *tiles_used;
    double *trace;
    int trace_tiles;
    int per_head;          /* ctx_lens [B][Hkv], block_table [B][Hkv][mbps], perm [B][Hkv][stride] */
    int order;             /* tile order: see visit_tile */
    const int32_t *perm;   /* order 2: [B][perm_stride] */
    int perm_stride;
    int next_item; /* work counter, protected by mu */
    pthread_mutex_t mu;
} job_t;

/* bf16 bit pattern -> double: the bf16 value is the top half of an fp32. */
static double widen_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16 bit pattern -> double, from the format's definition. */
static double widen_f16(uint16_t h) {
    int sign = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* the sequence (b, KV head g) reads: its own with per-head tables, else row b's */
static long seq_of(const job_t *J, int b, int g) {
    return J->per_head ? (long)b * J->Hkv + g : b;
}

/* index of cached row (b, kv head g, position j): returns -1 if the block id
   read from the table is out of range */
static long row_index(const job_t *J, int b, int g, int j) {
    if (J->block_size == 0)
        return ((long)b * J->Hkv + g) * J->max_ctx + j;
    int blk = J->block_table[seq_of(J, b, g) * J->max_blocks_per_seq + j / J->block_size];
    if (blk < 0 || blk >= J->num_blocks) return -1;
    return ((long)blk * J->Hkv + g) * J->block_size + (j % J->block_size);
}

/* Tile visited at step t (0-based) of sequence sq, which has nt tiles.  Section
   2.4 of the ART summary lets the sequence of tiles be reordered, e.g.
   recency-first or importance-first, with no approximation error since
   attention does not depend on the order, and has block 0 (the attention
   sink) evaluated before any termination.  Orders:
     0  ascending: 0, 1, ..., nt-1
     1  the sink, then the most recent first: 0, nt-1, nt-2, ..., 1
     2  the caller's list perm[sq][0..nt-1]: step 0 must name tile 0 and
        every later step a tile in 1..nt-1
   Returns -1 for a list entry that breaks those rules. */
static int visit_tile(const job_t *J, long sq, int nt, int t) {
    if (J->order == 0) return t;
    if (J->order == 1) return t == 0 ? 0 : nt - t;
    const int e = J->perm[sq * J->perm_stride + t];
    if (t == 0) return e == 0 ? 0 : -1;
    return (e >= 1 && e < nt) ? e : -1;
}

static void load_row(const job_t *J, const void *base, const uint16_t *scale, long row, double *dst) {
    const int d = J->d;
    if (J->kv_dtype == ODT_F32) {
        const float *p = (const float *)base + row * d;
        for (int i = 0; i < d; ++i) dst[i] = (double)p[i];
    } else if (J->kv_dtype == ODT_BF16) {
        const uint16_t *p = (const uint16_t *)base + row * d;
        for (int i = 0; i < d; ++i) dst[i] = widen_bf16(p[i]);
    } else if (J->kv_dtype == ODT_I8) {
        const int8_t *p = (const int8_t *)base + row * d;
        double s = widen_f16(scale[row]);
        for (int i = 0; i < d; ++i) dst[i] = (double)p[i] * s;
    } else {
        const uint8_t *p = (const uint8_t *)base + row * (d / 2);
        double s = widen_f16(scale[row]);
        for (int i = 0; i < d; ++i) {
            int nib = (i % 2 == 0) ? (p[i / 2] & 0x0f) : (p[i / 2] >> 4);
            int code = nib >= 8 ? nib - 16 : nib; /* two's complement, 4 bits */
            dst[i] = (double)code * s;
        }
    }
}

static double norm_of(const double *x, int n) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += x[i] * x[i];
    return sqrt(s);
}

/* one (batch row, query head) */
static int run_item(job_t *J, int b, int h, double *scratch) {
    const int d = J->d, T = J->tile, G = J->Hq / J->Hkv, g = h / G;
    const int P = d < 8 ? d : 8; /* probe dims 0..P-1 */
    double *q = scratch, *kr = q + d, *vr = kr + d, *acc = vr + d, *x = acc + d,
           *prev = x + 8, *s = prev + 8; /* s holds T scores */
    double *out = J->out + ((long)b * J->Hq + h) * d;
    int32_t *U_out = J->tiles_used + (long)b * J->Hq + h;
    const long sq = seq_of(J, b, g);
    const int n = J->ctx_lens[sq];
    const int nt = (n + T - 1) / T;

    /* widen the query */
    const long qoff = ((long)b * J->Hq + h) * d;
    for (int i = 0; i < d; ++i)
        q[i] = J->q_dtype == ODT_F32 ? (double)((const float *)J->q)[qoff + i]
                                     : widen_bf16(((const uint16_t *)J->q)[qoff + i]);
    for (int i = 0; i < d; ++i) { out[i] = 0.0; acc[i] = 0.0; }
    if (n == 0) { *U_out = 0; return 0; }

    const double sqrt_d = sqrt((double)d);
    double m = -INFINITY, l = 0.0, prev_norm = 0.0;
    int streak = 0, U = nt;

    for (int t = 0; t < nt; ++t) {
        const int pt = visit_tile(J, sq, nt, t); /* the tile of step t */
        if (pt < 0) return -1;
        const int j0 = pt * T, j1 = (j0 + T < n) ? j0 + T : n;
        /* scores of the tile, s_j = q.k_j / sqrt(d) */
        double tmax = -INFINITY;
        for (int j = j0; j < j1; ++j) {
            long r = row_index(J, b, g, j);
            if (r < 0) return -1;
            load_row(J, J->k, J->k_scale, r, kr);
            double dot = 0.0;
            for (int i = 0; i < d; ++i) dot += q[i] * kr[i];
            s[j - j0] = dot / sqrt_d;
            if (s[j - j0] > tmax) tmax = s[j - j0];
        }
        /* online softmax: new running max, rescale the old state */
        const double mt = tmax > m ? tmax : m;
        const double alpha = (m == -INFINITY) ? 0.0 : exp(m - mt);
        l *= alpha;
        for (int i = 0; i < d; ++i) acc[i] *= alpha;
        int kept = 0;
        for (int j = j0; j < j1; ++j) {
            const double p = exp(s[j - j0] - mt);
            l += p;
            if (J->v_skip_eps > 0.0 && p < J->v_skip_eps) continue; /* V row not used */
            long r = row_index(J, b, g, j);
            load_row(J, J->v, J->v_scale, r, vr);
            for (int i = 0; i < d; ++i) acc[i] += p * vr[i];
            ++kept;
        }
        m = mt;

        /* probe of the normalised running output */
        for (int i = 0; i < P; ++i) x[i] = acc[i] / l;
        const double xn = norm_of(x, P);
        double ds = NAN, dd = NAN;
        int stop = 0;
        if (t >= 1) {
            if (xn == 0.0 || prev_norm == 0.0) {
                ds = INFINITY;
                dd = INFINITY;
            } else {
                ds = fabs(xn - prev_norm) / prev_norm;
                double dot = 0.0;
                for (int i = 0; i < P; ++i) dot += x[i] * prev[i];
                dd = 1.0 - dot / (xn * prev_norm);
                if (dd < 0.0) dd = 0.0;
            }
            if (ds < J->eps_scale && dd < J->eps_dir) ++streak;
            else streak = 0;
            if (streak >= J->patience) stop = 1;
        }
        if (J->trace && t < J->trace_tiles) {
            double *tr = J->trace + (((long)b * J->Hq + h) * J->trace_tiles + t) * TRACE_FIELDS;
            tr[0] = m; tr[1] = l; tr[2] = ds; tr[3] = dd; tr[4] = streak;
            tr[5] = kept; tr[6] = xn; tr[7] = 1.0;
        }
        if (stop) { U = t + 1; break; }
        for (int i = 0; i < P; ++i) prev[i] = x[i];
        prev_norm = xn;
    }
    for (int i = 0; i < d; ++i) out[i] = acc[i] / l;
    *U_out = U;
    return 0;
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    double *scratch = (double *)malloc(sizeof(double) * (5 * (size_t)J->d + 16 + (size_t)J->tile));
    int bad = 0;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int it = J->next_item++;
        pthread_mutex_unlock(&J->mu);
        if (it >= J->B * J->Hq) break;
        if (run_item(J, it / J->Hq, it % J->Hq, scratch) != 0) bad = 1;
    }
    free(scratch);
    return bad ? (void *)1 : NULL;
}

/* Returns 0 on success, negative on a malformed argument, -100 if a block id
   read from the table lies outside [0, num_blocks) or an entry of a caller's
   tile order breaks the rules of visit_tile. */
int art_oracle_decode(int B, int Hq, int Hkv, int d, int q_dtype, int kv_dtype,
                      int block_size, int max_blocks_per_seq, int max_ctx, int num_blocks,
                      const void *q, const void *k, const void *v,
                      const uint16_t *k_scale, const uint16_t *v_scale,
                      const int32_t *block_table, const int32_t *ctx_lens,
                      int tile, double eps_scale, double eps_dir, int patience, double v_skip_eps,
                      double *out, int32_t *tiles_used,
                      double *trace, int trace_tiles, int nthreads,
                      int order, const int32_t *perm, int perm_stride, int per_head) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv) return -2;
    if (!q || !k || !v || !ctx_lens || !out || !tiles_used) return -1;
    if (q_dtype != ODT_F32 && q_dtype != ODT_BF16) return -3;
    if (kv_dtype < ODT_F32 || kv_dtype > ODT_I4) return -3;
    if ((kv_dtype == ODT_I8 || kv_dtype == ODT_I4) && (!k_scale || !v_scale)) return -1;
    if (kv_dtype == ODT_I4 && d % 2) return -2;
    if (tile <= 0 || patience < 1) return -5;
    if (order < 0 || order > 2) return -5;
    if (order == 2 && !perm) return -1;
    const long nseq = per_head ? (long)B * Hkv : B;
    for (long sq = 0; sq < nseq; ++sq) {
        long cap = block_size ? (long)max_blocks_per_seq * block_size : max_ctx;
        if (ctx_lens[sq] < 0 || ctx_lens[sq] > cap) return -2;
        if (order == 2 && (ctx_lens[sq] + tile - 1) / tile > perm_stride) return -2;
    }
    if (block_size && !block_table) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.d = d; J.q_dtype = q_dtype; J.kv_dtype = kv_dtype;
    J.block_size = block_size; J.max_blocks_per_seq = max_blocks_per_seq; J.max_ctx = max_ctx;
    J.num_blocks = num_blocks; J.q = q; J.k = k; J.v = v; J.k_scale = k_scale; J.v_scale = v_scale;
    J.block_table = block_table; J.ctx_lens = ctx_lens; J.tile = tile; J.patience = patience;
    J.eps_scale = eps_scale; J.eps_dir = eps_dir; J.v_skip_eps = v_skip_eps;
    J.out = out; J.tiles_used = tiles_used; J.trace = trace; J.trace_tiles = trace ? trace_tiles : 0;
    J.order = order; J.perm = perm; J.perm_stride = perm_stride; J.per_head = per_head != 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int bad = 0;
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
    for (int i = 0; i < nthreads; ++i) {
        void *r;
        pthread_join(th[i], &r);
        if (r) bad = 1;
    }
    pthread_mutex_destroy(&J.mu);
    return bad ? -100 : 0;
}

int art_oracle_trace_fields(void) { return TRACE_FIELDS; }

/* The widening of one fp16 bit pattern, exported so that the tests can check
   it against an independent IEEE binary16 decoder for every pattern. */
double art_oracle_widen_f16(int bits) { return widen_f16((uint16_t)bits); }
