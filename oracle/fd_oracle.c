/*
 * fd_oracle.c -- plain fp64 CPU oracle for split-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never links, loads or calls it, and this file includes nothing from it.
 *
 * What is computed (all in double precision, on the exact stored input
 * values: bf16 and fp32 elements are widened exactly, `scale` is widened
 * from the fp32 value the caller passes):
 *
 *   for every batch row b, query head h, query position t
 *     g   = h / (Hq / Hkv)                 GQA: consecutive query heads share
 *                                          one KV head (page "FlashDecoding
 *                                          算法原理与多GPU并行解码实战",
 *                                          engineering details, item 3)
 *     off = L_b - q_len                    the chunk's first absolute position
 *     J   = { j : 0 <= j <= off + t }      bottom-right causal visibility
 *                                          (page "ChunkedPrefill与FlashDecoding
 *                                          技术解析" §2.1: a chunk token sees
 *                                          itself and earlier positions; the
 *                                          cache already holds the chunk).
 *                                          For decode (q_len = 1) J = [0, L_b).
 *     s_j = scale * <q[b,h,t,:], k[b,g,j,:]>
 *     out = sum_j exp(s_j - M) v[b,g,j,:] / sum_j exp(s_j - M),  M = max s_j
 *     lse = M + ln sum_j exp(s_j - M)      natural log
 *     J empty -> out = 0, lse = -inf
 *
 * Three forms are provided, sharing only the input decoding helpers:
 *   orc_attention            the plain definition above;
 *   orc_attention_split      the split form: the key axis of each sequence is
 *                            cut into tiles, each tile gives a normalised
 *                            partial output with its max and sum, and the
 *                            partials are merged with the global-max
 *                            correction (page "FlashDecoding算法原理...",
 *                            algorithm section and multi-GPU step 3);
 *   orc_attention_sequential the running max / running sum / running output
 *                            rescaling over fixed blocks (page "ChunkedPrefill
 *                            与FlashDecoding技术解析" §3.1).
 * plus orc_merge_lse, the merge of given (o_s, lse_s) partials.
 *
 * Parity pins (tests that do not need a GPU) tie these functions to
 * hand-derived values, closed forms, invariants and a library attention
 * routine; see the test suite.
 *
 * Layouts (row-major, contiguous):
 *   q, out      [B, Hq, q_len, D]
 *   k, v        [B, Hkv, Lmax, D]
 *   cache_lens  [B]  int32, each in [0, Lmax]
 *   lse         [B, Hq, q_len]
 *   o_part      [B, Hq, q_len, S, D]    m_part, lse_part [B, Hq, q_len, S]
 * dtype: 0 = fp32, 1 = bf16 stored as raw uint16 bit patterns.
 * Return value: 0 on success, negative on bad arguments.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int B, Hq, Hkv, D, q_len, Lmax, dtype;
    const void *q, *k, *v;
    const int32_t *cache_lens;
    double scale;
} orc_problem;

/* bf16 is the upper half of an IEEE binary32 pattern: widening is exact. */
static double bf16_to_double(uint16_t x) {
    uint32_t bits = ((uint32_t)x) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int dtype, size_t idx) {
    if (dtype == 1) return bf16_to_double(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

static size_t q_index(const orc_problem *p, int b, int h, int t, int d) {
    return (((size_t)b * p->Hq + h) * p->q_len + t) * p->D + d;
}

static size_t kv_index(const orc_problem *p, int b, int g, int j, int d) {
    return (((size_t)b * p->Hkv + g) * p->Lmax + j) * p->D + d;
}

static int check_problem(const orc_problem *p) {
    if (p->B < 0 || p->Hq < 1 || p->Hkv < 1 || p->D < 1 || p->q_len < 1 || p->Lmax < 0) return -1;
    if (p->Hq % p->Hkv != 0) return -1;
    if (p->dtype != 0 && p->dtype != 1) return -1;
    for (int b = 0; b < p->B; ++b)
        if (p->cache_lens[b] < 0 || p->cache_lens[b] > p->Lmax) return -1;
    return 0;
}

/* Number of keys row (b, t) may attend to: keys 0 .. off+t, i.e. off+t+1 of
 * them, never more than the cache holds and never fewer than zero. */
static int visible_keys(const orc_problem *p, int b, int t) {
    int L = p->cache_lens[b];
    int n = L - p->q_len + t + 1;
    if (n > L) n = L;
    if (n < 0) n = 0;
    return n;
}

/* s_j = scale * <q_row, k_j> in double. */
static double score(const orc_problem *p, int b, int h, int t, int g, int j) {
    double acc = 0.0;
    for (int d = 0; d < p->D; ++d)
        acc += load_elem(p->q, p->dtype, q_index(p, b, h, t, d)) *
               load_elem(p->k, p->dtype, kv_index(p, b, g, j, d));
    return p->scale * acc;
}

/* ---------------------------------------------------------------------- */
/* Thread pool over independent (b, h, t) rows.                            */

typedef void (*row_fn)(void *ctx, long row, double *scratch);

typedef struct {
    row_fn fn;
    void *ctx;
    long nrows;
    long next;
    size_t scratch_len;
    pthread_mutex_t lock;
} row_pool;

static void *row_worker(void *arg) {
    row_pool *pool = (row_pool *)arg;
    double *scratch = (double *)malloc((pool->scratch_len + 1) * sizeof(double));
    if (!scratch) return (void *)1;
    for (;;) {
        pthread_mutex_lock(&pool->lock);
        long row = pool->next++;
        pthread_mutex_unlock(&pool->lock);
        if (row >= pool->nrows) break;
        pool->fn(pool->ctx, row, scratch);
    }
    free(scratch);
    return NULL;
}

static int run_rows(row_fn fn, void *ctx, long nrows, size_t scratch_len, int nthreads) {
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((long)nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    row_pool pool = {fn, ctx, nrows, 0, scratch_len, PTHREAD_MUTEX_INITIALIZER};
    pthread_t tid[256];
    int started = 0, failed = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, row_worker, &pool) != 0) { failed = 1; break; }
        ++started;
    }
    if (started == 0) return -2;
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(tid[i], &ret);
        if (ret) failed = 1;
    }
    return failed ? -2 : 0;
}

static void split_row(const orc_problem *p, long row, int *b, int *h, int *t) {
    *t = (int)(row % p->q_len);
    long bh = row / p->q_len;
    *h = (int)(bh % p->Hq);
    *b = (int)(bh / p->Hq);
}

/* ---------------------------------------------------------------------- */
/* Plain definition.                                                       */

typedef struct {
    const orc_problem *p;
    double *out, *lse;
} direct_ctx;

static void direct_row(void *vctx, long row, double *s) {
    direct_ctx *c = (direct_ctx *)vctx;
    const orc_problem *p = c->p;
    int b, h, t;
    split_row(p, row, &b, &h, &t);
    int g = h / (p->Hq / p->Hkv);
    int n = visible_keys(p, b, t);
    double *o = c->out + (size_t)row * p->D;
    for (int d = 0; d < p->D; ++d) o[d] = 0.0;
    if (n == 0) {
        c->lse[row] = -INFINITY;
        return;
    }
    double M = -INFINITY;
    for (int j = 0; j < n; ++j) {
        s[j] = score(p, b, h, t, g, j);
        if (s[j] > M) M = s[j];
    }
    double Z = 0.0;
    for (int j = 0; j < n; ++j) Z += exp(s[j] - M);
    for (int j = 0; j < n; ++j) {
        double w = exp(s[j] - M) / Z;
        for (int d = 0; d < p->D; ++d) o[d] += w * load_elem(p->v, p->dtype, kv_index(p, b, g, j, d));
    }
    c->lse[row] = M + log(Z);
}

int orc_attention(int B, int Hq, int Hkv, int D, int q_len, int Lmax, int dtype,
                  const void *q, const void *k, const void *v, const int32_t *cache_lens,
                  double scale, double *out, double *lse, int nthreads) {
    orc_problem p = {B, Hq, Hkv, D, q_len, Lmax, dtype, q, k, v, cache_lens, scale};
    if (check_problem(&p)) return -1;
    direct_ctx c = {&p, out, lse};
    return run_rows(direct_row, &c, (long)B * Hq * q_len, (size_t)Lmax, nthreads);
}

/* ---------------------------------------------------------------------- */
/* Split form: per-tile partial softmax, then the global-max merge.        */

typedef struct {
    const orc_problem *p;
    int num_splits; /* > 0: tile = ceil(L_b / num_splits) for each sequence */
    int tile_len;   /* used when num_splits == 0 */
    int S;          /* partial slots per row */
    double *o_part, *m_part, *lse_part, *out, *lse;
} split_ctx;

static void split_row_fn(void *vctx, long row, double *s) {
    split_ctx *c = (split_ctx *)vctx;
    const orc_problem *p = c->p;
    int b, h, t;
    split_row(p, row, &b, &h, &t);
    int g = h / (p->Hq / p->Hkv);
    int L = p->cache_lens[b];
    int n = visible_keys(p, b, t);
    /* Tile length: ceil(L / num_chunks) when a chunk count is given, as in the
     * chunked split of the algorithm section; otherwise a fixed tile. */
    int T = c->num_splits > 0 ? (L + c->num_splits - 1) / c->num_splits : c->tile_len;
    if (T < 1) T = 1;
    double *mp = c->m_part + (size_t)row * c->S;
    double *lp = c->lse_part + (size_t)row * c->S;
    double *op = c->o_part + (size_t)row * c->S * p->D;
    for (int i = 0; i < c->S; ++i) {
        mp[i] = -INFINITY;
        lp[i] = -INFINITY;
        for (int d = 0; d < p->D; ++d) op[(size_t)i * p->D + d] = 0.0;
    }
    /* Step 1: each tile [i*T, (i+1)*T) of the cache, restricted to the keys
     * this row may see, gives m_i (tile max), l_i (sum of exp(s - m_i)) and
     * o_i = sum exp(s - m_i) v / l_i. */
    int num_tiles = (L + T - 1) / T;
    for (int i = 0; i < num_tiles && i < c->S; ++i) {
        int lo = i * T;
        int hi = lo + T < n ? lo + T : n;
        if (hi <= lo) continue; /* no visible key: m = lse = -inf, o = 0 */
        double m = -INFINITY;
        for (int j = lo; j < hi; ++j) {
            s[j - lo] = score(p, b, h, t, g, j);
            if (s[j - lo] > m) m = s[j - lo];
        }
        double l = 0.0;
        for (int j = lo; j < hi; ++j) l += exp(s[j - lo] - m);
        for (int j = lo; j < hi; ++j) {
            double w = exp(s[j - lo] - m) / l;
            for (int d = 0; d < p->D; ++d)
                op[(size_t)i * p->D + d] += w * load_elem(p->v, p->dtype, kv_index(p, b, g, j, d));
        }
        mp[i] = m;
        lp[i] = m + log(l);
    }
    /* Step 2: global max over the tile maxima. */
    double mg = -INFINITY;
    for (int i = 0; i < c->S; ++i)
        if (mp[i] > mg) mg = mp[i];
    double *o = c->out + (size_t)row * p->D;
    for (int d = 0; d < p->D; ++d) o[d] = 0.0;
    if (mg == -INFINITY) {
        c->lse[row] = -INFINITY;
        return;
    }
    /* Step 3: out = sum_i o_i e^{m_i - mg} l_i / sum_i e^{m_i - mg} l_i, where
     * l_i = e^{lse_i - m_i} is tile i's softmax denominator (the merge of the
     * multi-GPU section, reading its per-tile weight as that denominator). */
    double den = 0.0;
    for (int i = 0; i < c->S; ++i) {
        if (mp[i] == -INFINITY) continue;
        double li = exp(lp[i] - mp[i]);
        double wi = exp(mp[i] - mg) * li;
        den += wi;
        for (int d = 0; d < p->D; ++d) o[d] += wi * op[(size_t)i * p->D + d];
    }
    for (int d = 0; d < p->D; ++d) o[d] /= den;
    c->lse[row] = mg + log(den);
}

int orc_attention_split(int B, int Hq, int Hkv, int D, int q_len, int Lmax, int dtype,
                        const void *q, const void *k, const void *v, const int32_t *cache_lens,
                        double scale, int num_splits, int tile_len, int S,
                        double *o_part, double *m_part, double *lse_part,
                        double *out, double *lse, int nthreads) {
    orc_problem p = {B, Hq, Hkv, D, q_len, Lmax, dtype, q, k, v, cache_lens, scale};
    if (check_problem(&p)) return -1;
    if (S < 1 || num_splits < 0 || (num_splits == 0 && tile_len < 1)) return -1;
    /* Every tile must have a slot. */
    for (int b = 0; b < B; ++b) {
        int L = cache_lens[b];
        int T = num_splits > 0 ? (L + num_splits - 1) / num_splits : tile_len;
        if (T < 1) T = 1;
        if ((L + T - 1) / T > S) return -1;
    }
    split_ctx c = {&p, num_splits, tile_len, S, o_part, m_part, lse_part, out, lse};
    return run_rows(split_row_fn, &c, (long)B * Hq * q_len, (size_t)Lmax, nthreads);
}

/* ---------------------------------------------------------------------- */
/* Split form over explicit key ranges: slot i of the rows of (b, g) covers  */
/* keys [lo, hi) of range arrays [B][Hkv][S] (lo >= hi: an empty slot).      */
/* Each slot's partial is the definition over its visible keys; the output */
/* is their merge.  Any disjoint ranges covering each row's visible keys    */
/* give the attention itself.                                               */

typedef struct {
    const orc_problem *p;
    int S;
    const int32_t *lo, *hi;
    double *o_part, *m_part, *lse_part, *out, *lse;
} range_ctx;

static void range_row_fn(void *vctx, long row, double *s) {
    range_ctx *c = (range_ctx *)vctx;
    const orc_problem *p = c->p;
    int b, h, t;
    split_row(p, row, &b, &h, &t);
    const int g = h / (p->Hq / p->Hkv);
    const int n = visible_keys(p, b, t);
    const size_t pair = ((size_t)b * p->Hkv + g) * c->S;
    double *mp = c->m_part + (size_t)row * c->S;
    double *lp = c->lse_part + (size_t)row * c->S;
    double *op = c->o_part + (size_t)row * c->S * p->D;
    double *o = c->out + (size_t)row * p->D;
    for (int d = 0; d < p->D; ++d) o[d] = 0.0;
    double M = -INFINITY;
    for (int i = 0; i < c->S; ++i) {
        int lo = c->lo[pair + i], hi = c->hi[pair + i];
        if (hi > n) hi = n;
        mp[i] = -INFINITY;
        lp[i] = -INFINITY;
        for (int d = 0; d < p->D; ++d) op[(size_t)i * p->D + d] = 0.0;
        if (lo < 0) lo = 0;
        if (hi <= lo) continue;
        double m = -INFINITY;
        for (int j = lo; j < hi; ++j) {
            s[j - lo] = score(p, b, h, t, g, j);
            m = s[j - lo] > m ? s[j - lo] : m;
        }
        double z = 0.0;
        for (int j = lo; j < hi; ++j) z += exp(s[j - lo] - m);
        for (int j = lo; j < hi; ++j) {
            const double w = exp(s[j - lo] - m) / z;
            for (int d = 0; d < p->D; ++d)
                op[(size_t)i * p->D + d] += w * load_elem(p->v, p->dtype, kv_index(p, b, g, j, d));
        }
        mp[i] = m;
        lp[i] = m + log(z);
        M = lp[i] > M ? lp[i] : M;
    }
    if (M == -INFINITY) {
        c->lse[row] = -INFINITY;
        return;
    }
    /* exp(LSE) = sum_i exp(lse_i); out = sum_i exp(lse_i - LSE) o_i. */
    double z = 0.0;
    for (int i = 0; i < c->S; ++i)
        if (lp[i] != -INFINITY) z += exp(lp[i] - M);
    for (int i = 0; i < c->S; ++i) {
        if (lp[i] == -INFINITY) continue;
        const double w = exp(lp[i] - M) / z;
        for (int d = 0; d < p->D; ++d) o[d] += w * op[(size_t)i * p->D + d];
    }
    c->lse[row] = M + log(z);
}

int orc_attention_ranges(int B, int Hq, int Hkv, int D, int q_len, int Lmax, int dtype,
                         const void *q, const void *k, const void *v, const int32_t *cache_lens,
                         double scale, int S, const int32_t *lo, const int32_t *hi,
                         double *o_part, double *m_part, double *lse_part,
                         double *out, double *lse, int nthreads) {
    orc_problem p = {B, Hq, Hkv, D, q_len, Lmax, dtype, q, k, v, cache_lens, scale};
    if (check_problem(&p)) return -1;
    if (S < 1 || !lo || !hi) return -1;
    for (size_t i = 0; i < (size_t)B * Hkv * S; ++i)
        if (lo[i] < hi[i] && (lo[i] < 0 || hi[i] > Lmax)) return -1;
    range_ctx c = {&p, S, lo, hi, o_part, m_part, lse_part, out, lse};
    return run_rows(range_row_fn, &c, (long)B * Hq * q_len, (size_t)Lmax, nthreads);
}

/* ---------------------------------------------------------------------- */
/* Sequential form: running max, running sum and running output, rescaled  */
/* block by block.                                                         */

typedef struct {
    const orc_problem *p;
    int block;
    double *out, *lse;
} seq_ctx;

static void seq_row(void *vctx, long row, double *s) {
    seq_ctx *c = (seq_ctx *)vctx;
    const orc_problem *p = c->p;
    int b, h, t;
    split_row(p, row, &b, &h, &t);
    int g = h / (p->Hq / p->Hkv);
    int n = visible_keys(p, b, t);
    double *acc = s;          /* running output, D values */
    double *sc = s + p->D;    /* scores of the current block */
    double *o = c->out + (size_t)row * p->D;
    double gmax = -INFINITY, gsum = 0.0;
    for (int d = 0; d < p->D; ++d) acc[d] = 0.0;
    for (int lo = 0; lo < n; lo += c->block) {
        int hi = lo + c->block < n ? lo + c->block : n;
        double bmax = -INFINITY;
        for (int j = lo; j < hi; ++j) {
            sc[j - lo] = score(p, b, h, t, g, j);
            if (sc[j - lo] > bmax) bmax = sc[j - lo];
        }
        double nmax = gmax > bmax ? gmax : bmax;
        double diff = exp(gmax - nmax); /* gmax = -inf on the first block: 0 */
        for (int d = 0; d < p->D; ++d) acc[d] *= diff;
        gsum *= diff;
        for (int j = lo; j < hi; ++j) {
            double e = exp(sc[j - lo] - nmax);
            for (int d = 0; d < p->D; ++d) acc[d] += e * load_elem(p->v, p->dtype, kv_index(p, b, g, j, d));
            gsum += e;
        }
        gmax = nmax;
    }
    if (n == 0) {
        for (int d = 0; d < p->D; ++d) o[d] = 0.0;
        c->lse[row] = -INFINITY;
        return;
    }
    for (int d = 0; d < p->D; ++d) o[d] = acc[d] / gsum;
    c->lse[row] = gmax + log(gsum);
}

int orc_attention_sequential(int B, int Hq, int Hkv, int D, int q_len, int Lmax, int dtype,
                             const void *q, const void *k, const void *v, const int32_t *cache_lens,
                             double scale, int block, double *out, double *lse, int nthreads) {
    orc_problem p = {B, Hq, Hkv, D, q_len, Lmax, dtype, q, k, v, cache_lens, scale};
    if (check_problem(&p)) return -1;
    if (block < 1) return -1;
    seq_ctx c = {&p, block, out, lse};
    return run_rows(seq_row, &c, (long)B * Hq * q_len, (size_t)D + (size_t)block, nthreads);
}

/* ---------------------------------------------------------------------- */
/* Merge of given partials: exp(LSE) = sum_s exp(lse_s),                    */
/* out = sum_s exp(lse_s - LSE) o_s.  Slots with lse_s = -inf are empty and */
/* their o_s is not read.  No finite slot: out = 0, LSE = -inf.             */

int orc_merge_lse(long rows, int S, int D, const double *o_part, const double *lse_part,
                  double *out, double *lse) {
    if (rows < 0 || S < 1 || D < 1) return -1;
    for (long r = 0; r < rows; ++r) {
        const double *lp = lse_part + (size_t)r * S;
        const double *op = o_part + (size_t)r * S * D;
        double *o = out + (size_t)r * D;
        double M = -INFINITY;
        for (int i = 0; i < S; ++i)
            if (lp[i] > M) M = lp[i];
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double Z = 0.0;
        for (int i = 0; i < S; ++i)
            if (lp[i] != -INFINITY) Z += exp(lp[i] - M);
        double LSE = M + log(Z);
        for (int i = 0; i < S; ++i) {
            if (lp[i] == -INFINITY) continue;
            double w = exp(lp[i] - LSE);
            for (int d = 0; d < D; ++d) o[d] += w * op[(size_t)i * D + d];
        }
        lse[r] = LSE;
    }
    return 0;
}
