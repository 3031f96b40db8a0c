/*
 * Oracle for the chunked spatio-temporal attention queue step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, fp64 CPU statement
 * of what the GPU path must compute.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark load it; the product library never
 * does, and the two share no code, headers or tables.
 *
 * What is computed (cited by page title and section):
 *
 *  - "双重并行：让AI视频生成突破时长限制" (techwalker write-up of DualParal,
 *    arXiv:2505.21070), section 二 (FIFO queue and block-wise denoising): the
 *    video is split into fixed-size,
 *    non-overlapping temporal chunks that sit in a FIFO queue and are all
 *    processed in one step, fed from the tail to the head.
 *  - same page, section 三 (feature cache): while chunk B_{i+1} is processed
 *    its self-attention K/V are stored, and the next chunk processed (B_i)
 *    reuses them instead of re-concatenating that chunk; only self-attention
 *    uses the cache, cross-attention and the FFN stay per chunk.
 *  - "视频扩散模型：核心技术挑战与前沿进展" (intelliparadigm survey),
 *    section 2.1, item 2: spatio-temporal attention attends jointly over all
 *    tokens of all frames in the window, at quadratic cost.
 *
 * Reading used here.  Chunk c of the call is the c-th chunk in processing
 * order; its "predecessor" is chunk c-1 (the chunk processed just before it,
 * the page's B_{i+1}).  Chunk 0 has no predecessor and so a zero-length cache.
 * For query row r of chunk c and head h, the key/value set is
 *     R_c = [predecessor rows 0..L-1 (if c >= 1)] ++ [own rows 0..L-1]
 * and the output is plain softmax attention over R_c:
 *     s_j = scale * <q, k_j>,  O = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s)
 * with no mask inside R_c.  The predecessor rows come either from a separate
 * cache buffer (slot c holds chunk c-1's K then V) or, when no cache buffer is
 * given, straight from chunk c-1's own K/V.
 *
 * Window step (same page, section 三, the form the cache is introduced for).
 * Processing a window of three neighbouring chunks [B_{i-1}, B_i, B_{i+1}]
 * would repeat B_{i+1}, which the window processed just before already
 * handled; its self-attention K/V is cached there and reused, so the window's
 * own input shrinks to [B_{i-1}, B_i].  Reading used here, with chunks indexed
 * in processing order as above: window c is centred on chunk c (B_i); its
 * queries are the rows of chunk c and of chunk c+1 (B_{i-1}, the next chunk
 * to be processed), 2L rows, or L rows for the last window, which has no chunk
 * c+1; its key/value set is
 *     W_c = [predecessor rows (chunk c-1, if c >= 1)] ++ [own rows of chunk c]
 *           ++ [own rows of chunk c+1 (if c+1 < n)]
 * and each query row gets plain softmax attention over W_c, as above.  The
 * output of window c holds its 2L query rows: out[c][0] = chunk c's rows,
 * out[c][1] = chunk c+1's rows (absent for the last window).
 *
 * Streaming queue (same page, section 二: new noisy chunks enter at the tail,
 * clean ones leave at the head, the queue is processed from tail to head, so
 * the video can grow without bound).  The chunks live in a ring of S slots;
 * with the live chunks listed in processing order (c = 0 is the tail, the
 * newest), chunk c sits in slot (tail - c) mod S, and its predecessor (chunk
 * c-1, the next newer one, processed just before it) in slot
 * (tail - c + 1) mod S, read in place.  Each live chunk then attends over R_c
 * exactly as above.
 *
 * Precision.  Every input element is widened exactly to fp64 (bf16 and fp32
 * both embed exactly); scores, exponentials, sums and the weighted sum are
 * fp64, the dot product summed in increasing dimension order.  Two passes per
 * row: all scores first, then the normalised weighted sum.  No tiling, no
 * running maximum.
 *
 * Layouts (row-major, element offsets):
 *   q, k, v, out      [n_chunks][L][H][D]
 *   kv_cache          [n_chunks][2][L][H][D]   (slot c: K of c-1, then V of c-1)
 *   window out        [n_chunks][2][L][H][D]   (window c: chunk c, then chunk c+1)
 *   ring q, k, v, out [S][L][H][D]             (slot p; chunk c of the queue in
 *                                               slot (tail - c) mod S)
 *   full attention    q/out [batch][Lq][H][D],  k/v batch b at b*kv_batch_stride,
 *                     each [Lkv][H][D]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2 };
enum { ORACLE_SRC_PRED = 0, ORACLE_SRC_OWN = 1 };

/* Widen element i of an array of the given storage type to fp64. */
static double load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    return ((const double *)base)[i];
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Size of R_c. */
int64_t oracle_kv_set_size(int64_t chunk_len, int64_t c)
{
    return c >= 1 ? 2 * chunk_len : chunk_len;
}

/*
 * The key/value set R_c of chunk c, entry by entry: which source it is read
 * from (predecessor or own), which chunk's K/V it is, and the token row in that
 * chunk.  This is the integer map the GPU plan must reproduce bit for bit.
 */
int64_t oracle_index_map(int64_t chunk_len, int64_t n_chunks, int64_t c,
                         int64_t *src, int64_t *chunk, int64_t *row)
{
    if (c < 0 || c >= n_chunks || chunk_len < 0)
        return -1;
    int64_t j = 0;
    if (c >= 1) {
        for (int64_t r = 0; r < chunk_len; ++r, ++j) {
            src[j] = ORACLE_SRC_PRED;
            chunk[j] = c - 1;
            row[j] = r;
        }
    }
    for (int64_t r = 0; r < chunk_len; ++r, ++j) {
        src[j] = ORACLE_SRC_OWN;
        chunk[j] = c;
        row[j] = r;
    }
    return j;
}

/* Element offsets of the K and V row for entry j of R_c, head h, dim 0. */
static void kv_offsets(int64_t j, int64_t c, int64_t L, int64_t H, int64_t D,
                       int has_cache, int64_t *k_off, int64_t *v_off,
                       int *from_cache)
{
    int64_t lc = c >= 1 ? L : 0;
    if (j < lc) {
        if (has_cache) {
            /* cache slot c: [2][L][H][D], K first then V */
            *k_off = ((c * 2 + 0) * L + j) * H * D;
            *v_off = ((c * 2 + 1) * L + j) * H * D;
            *from_cache = 1;
        } else {
            /* predecessor read in place from chunk c-1 */
            *k_off = ((c - 1) * L + j) * H * D;
            *v_off = *k_off;
            *from_cache = 0;
        }
    } else {
        *k_off = (c * L + (j - lc)) * H * D;
        *v_off = *k_off;
        *from_cache = 0;
    }
}

/*
 * Attention of one query row (q_off: element offset of (token, head, 0) in q)
 * over nk key/value rows whose element offsets are given by the callback data.
 * Writes the D outputs to out; when probs is non-NULL also writes the nk
 * softmax weights.  s is scratch of nk doubles.
 */
typedef struct {
    const void *k, *v, *ck;
    int64_t c, L, H, D, h;
    int has_cache;
    /* full attention */
    int64_t kv_base;
    int full;
    /* window step: W_c as listed by its index map */
    const int64_t *map_src, *map_chunk, *map_row;
    int window;
} kv_source;

static void window_entry(const void *k, const void *v, const void *kv_cache, int64_t L,
                         int64_t H, int64_t D, int64_t c, int64_t h, int64_t src,
                         int64_t chunk, int64_t row, const void **kb, int64_t *ko,
                         const void **vb, int64_t *vo);

static void row_kv(const kv_source *src, int64_t j, const void **kb, int64_t *ko,
                   const void **vb, int64_t *vo)
{
    if (src->window) {
        window_entry(src->k, src->v, src->ck, src->L, src->H, src->D, src->c, src->h,
                     src->map_src[j], src->map_chunk[j], src->map_row[j], kb, ko, vb, vo);
        return;
    }
    if (src->full) {
        *kb = src->k;
        *vb = src->v;
        *ko = src->kv_base + (j * src->H + src->h) * src->D;
        *vo = *ko;
        return;
    }
    int64_t k_off, v_off;
    int from_cache;
    kv_offsets(j, src->c, src->L, src->H, src->D, src->has_cache, &k_off, &v_off,
               &from_cache);
    k_off += src->h * src->D;
    v_off += src->h * src->D;
    if (from_cache) {
        *kb = src->ck;
        *vb = src->ck;
    } else {
        *kb = src->k;
        *vb = src->v;
    }
    *ko = k_off;
    *vo = v_off;
}

static void attend_row(int dtype, const void *q, int64_t q_off, const kv_source *src,
                       int64_t nk, double scale, double *s, double *out, double *probs)
{
    const int64_t D = src->D;
    /* pass 1: scores */
    for (int64_t j = 0; j < nk; ++j) {
        const void *kb, *vb;
        int64_t ko, vo;
        row_kv(src, j, &kb, &ko, &vb, &vo);
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += load_elem(q, dtype, q_off + d) * load_elem(kb, dtype, ko + d);
        s[j] = scale * acc;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j)
        if (s[j] > m)
            m = s[j];
    double z = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    /* pass 2: normalised weighted sum of V */
    for (int64_t d = 0; d < D; ++d)
        out[d] = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        const void *kb, *vb;
        int64_t ko, vo;
        row_kv(src, j, &kb, &ko, &vb, &vo);
        double w = s[j] / z;
        if (probs)
            probs[j] = w;
        for (int64_t d = 0; d < D; ++d)
            out[d] += w * load_elem(vb, dtype, vo + d);
    }
}

static kv_source queue_source(const void *k, const void *v, const void *kv_cache,
                              int64_t c, int64_t h, int64_t L, int64_t H, int64_t D)
{
    kv_source src;
    memset(&src, 0, sizeof src);
    src.k = k;
    src.v = v;
    src.ck = kv_cache;
    src.c = c;
    src.h = h;
    src.L = L;
    src.H = H;
    src.D = D;
    src.has_cache = kv_cache != NULL;
    return src;
}

/*
 * Queue step over selected rows.  rows holds n_rows triples (chunk, head, row);
 * out receives n_rows x D doubles.  Returns 0, or -1 on a bad argument.
 */
int oracle_queue_rows(int dtype, const void *q, const void *k, const void *v,
                      const void *kv_cache, int64_t L, int64_t n_chunks, int64_t H,
                      int64_t D, double scale, const int64_t *rows, int64_t n_rows,
                      double *out)
{
    if (L <= 0 || n_chunks <= 0 || H <= 0 || D <= 0)
        return -1;
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t c = rows[3 * i], h = rows[3 * i + 1], r = rows[3 * i + 2];
        if (c < 0 || c >= n_chunks || h < 0 || h >= H || r < 0 || r >= L)
            return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * 2 * L);
        if (!s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < n_rows; ++i) {
                int64_t c = rows[3 * i], h = rows[3 * i + 1], r = rows[3 * i + 2];
                kv_source src = queue_source(k, v, kv_cache, c, h, L, H, D);
                int64_t q_off = ((c * L + r) * H + h) * D;
                attend_row(dtype, q, q_off, &src, oracle_kv_set_size(L, c), scale, s,
                           out + i * D, NULL);
            }
            free(s);
        }
    }
    return bad ? -2 : 0;
}

/* Whole queue step: out is [n_chunks][L][H][D] doubles. */
int oracle_queue_step(int dtype, const void *q, const void *k, const void *v,
                      const void *kv_cache, int64_t L, int64_t n_chunks, int64_t H,
                      int64_t D, double scale, double *out)
{
    if (L <= 0 || n_chunks <= 0 || H <= 0 || D <= 0)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * 2 * L);
        if (!s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for collapse(3) schedule(dynamic, 4)
            for (int64_t c = 0; c < n_chunks; ++c)
                for (int64_t r = 0; r < L; ++r)
                    for (int64_t h = 0; h < H; ++h) {
                        kv_source src = queue_source(k, v, kv_cache, c, h, L, H, D);
                        int64_t off = ((c * L + r) * H + h) * D;
                        attend_row(dtype, q, off, &src, oracle_kv_set_size(L, c), scale,
                                   s, out + off, NULL);
                    }
            free(s);
        }
    }
    return bad ? -2 : 0;
}

/* Softmax weights of one query row over R_c, in index-map order. */
int oracle_queue_probs(int dtype, const void *q, const void *k, const void *v,
                       const void *kv_cache, int64_t L, int64_t n_chunks, int64_t H,
                       int64_t D, double scale, int64_t c, int64_t h, int64_t r,
                       double *probs, double *out_row)
{
    if (L <= 0 || c < 0 || c >= n_chunks || h < 0 || h >= H || r < 0 || r >= L)
        return -1;
    int64_t nk = oracle_kv_set_size(L, c);
    double *s = (double *)malloc(sizeof(double) * nk);
    if (!s)
        return -2;
    kv_source src = queue_source(k, v, kv_cache, c, h, L, H, D);
    attend_row(dtype, q, ((c * L + r) * H + h) * D, &src, nk, scale, s, out_row, probs);
    free(s);
    return 0;
}

/*
 * Full (non-chunked) attention, also used for per-chunk cross-attention to a
 * shared text K/V (kv_batch_stride = 0).  rows: n_rows triples (batch, head,
 * query row); out: n_rows x D.  Pass rows = NULL to compute every row, in
 * which case out is [batch][Lq][H][D].
 */
int oracle_full_rows(int dtype, const void *q, const void *k, const void *v,
                     int64_t batch, int64_t lq, int64_t lkv, int64_t kv_batch_stride,
                     int64_t H, int64_t D, double scale, const int64_t *rows,
                     int64_t n_rows, double *out)
{
    if (batch <= 0 || lq <= 0 || lkv <= 0 || H <= 0 || D <= 0 || kv_batch_stride < 0)
        return -1;
    int all = rows == NULL;
    int64_t total = all ? batch * lq * H : n_rows;
    if (!all)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t b = rows[3 * i], h = rows[3 * i + 1], r = rows[3 * i + 2];
            if (b < 0 || b >= batch || h < 0 || h >= H || r < 0 || r >= lq)
                return -1;
        }
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * lkv);
        if (!s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < total; ++i) {
                int64_t b, h, r;
                if (all) {
                    h = i % H;
                    r = (i / H) % lq;
                    b = i / (H * lq);
                } else {
                    b = rows[3 * i];
                    h = rows[3 * i + 1];
                    r = rows[3 * i + 2];
                }
                kv_source src;
                memset(&src, 0, sizeof src);
                src.full = 1;
                src.k = k;
                src.v = v;
                src.H = H;
                src.D = D;
                src.h = h;
                src.kv_base = b * kv_batch_stride;
                int64_t q_off = ((b * lq + r) * H + h) * D;
                double *dst = all ? out + q_off : out + i * D;
                attend_row(dtype, q, q_off, &src, lkv, scale, s, dst, NULL);
            }
            free(s);
        }
    }
    return bad ? -2 : 0;
}

/* ---- window step ------------------------------------------------------- */

/* Query rows of window c: chunk c, and chunk c+1 when it exists. */
int64_t oracle_window_q_rows(int64_t chunk_len, int64_t n_chunks, int64_t c)
{
    return c + 1 < n_chunks ? 2 * chunk_len : chunk_len;
}

/* Size of W_c. */
int64_t oracle_window_kv_set_size(int64_t chunk_len, int64_t n_chunks, int64_t c)
{
    int64_t m = chunk_len;                 /* own rows of chunk c */
    if (c >= 1)
        m += chunk_len;                    /* cached rows of chunk c-1 */
    if (c + 1 < n_chunks)
        m += chunk_len;                    /* own rows of chunk c+1 */
    return m;
}

/* W_c entry by entry: (source, chunk, token row), in the order stated above. */
int64_t oracle_window_index_map(int64_t chunk_len, int64_t n_chunks, int64_t c,
                                int64_t *src, int64_t *chunk, int64_t *row)
{
    if (c < 0 || c >= n_chunks || chunk_len < 0)
        return -1;
    int64_t j = 0;
    if (c >= 1)
        for (int64_t r = 0; r < chunk_len; ++r, ++j) {
            src[j] = ORACLE_SRC_PRED;
            chunk[j] = c - 1;
            row[j] = r;
        }
    for (int64_t r = 0; r < chunk_len; ++r, ++j) {
        src[j] = ORACLE_SRC_OWN;
        chunk[j] = c;
        row[j] = r;
    }
    if (c + 1 < n_chunks)
        for (int64_t r = 0; r < chunk_len; ++r, ++j) {
            src[j] = ORACLE_SRC_OWN;
            chunk[j] = c + 1;
            row[j] = r;
        }
    return j;
}

/*
 * Element offsets (head h, dim 0) of W_c entry j: a predecessor entry comes
 * from cache slot c when a cache buffer is given (K half, then V half), else
 * from chunk c-1's own K/V; an own entry from its chunk's K/V.
 */
static void window_entry(const void *k, const void *v, const void *kv_cache, int64_t L,
                         int64_t H, int64_t D, int64_t c, int64_t h, int64_t src,
                         int64_t chunk, int64_t row, const void **kb, int64_t *ko,
                         const void **vb, int64_t *vo)
{
    if (src == ORACLE_SRC_PRED && kv_cache) {
        *kb = kv_cache;
        *vb = kv_cache;
        *ko = (((c * 2 + 0) * L + row) * H + h) * D;
        *vo = (((c * 2 + 1) * L + row) * H + h) * D;
    } else {
        *kb = k;
        *vb = v;
        *ko = ((chunk * L + row) * H + h) * D;
        *vo = *ko;
    }
}

/*
 * Window step over selected rows: rows holds n_rows triples (window c, head h,
 * row r) with r < oracle_window_q_rows(L, n, c); row r is chunk c's token r
 * for r < L and chunk c+1's token r-L otherwise.  out: n_rows x D doubles.
 * Pass rows = NULL for every row; out is then [n][2][L][H][D] with the absent
 * half of the last window set to NaN.
 */
int oracle_window_rows(int dtype, const void *q, const void *k, const void *v,
                       const void *kv_cache, int64_t L, int64_t n, int64_t H, int64_t D,
                       double scale, const int64_t *rows, int64_t n_rows, double *out)
{
    if (L <= 0 || n <= 0 || H <= 0 || D <= 0)
        return -1;
    const int all = rows == NULL;
    if (!all)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t c = rows[3 * i], h = rows[3 * i + 1], r = rows[3 * i + 2];
            if (c < 0 || c >= n || h < 0 || h >= H || r < 0 ||
                r >= oracle_window_q_rows(L, n, c))
                return -1;
        }
    const int64_t total = all ? n * 2 * L * H : n_rows;
    const int64_t max_nk = 3 * L;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * max_nk);
        int64_t *map = (int64_t *)malloc(sizeof(int64_t) * 3 * max_nk);
        if (!s || !map) {
#pragma omp atomic write
            bad = 1;
        } else {
            int64_t map_c = -1, nk = 0;
#pragma omp for schedule(dynamic, 8)
            for (int64_t i = 0; i < total; ++i) {
                int64_t c, h, r;
                double *dst;
                if (all) {
                    /* out[c][half][row][h][:] */
                    h = i % H;
                    const int64_t rr = (i / H) % L, half = (i / (H * L)) % 2;
                    c = i / (H * L * 2);
                    r = half * L + rr;
                    dst = out + i * D;
                    if (r >= oracle_window_q_rows(L, n, c)) {
                        for (int64_t d = 0; d < D; ++d)
                            dst[d] = NAN;
                        continue;
                    }
                } else {
                    c = rows[3 * i];
                    h = rows[3 * i + 1];
                    r = rows[3 * i + 2];
                    dst = out + i * D;
                }
                if (c != map_c) {
                    nk = oracle_window_index_map(L, n, c, map, map + max_nk, map + 2 * max_nk);
                    map_c = c;
                }
                const int64_t q_chunk = r < L ? c : c + 1;
                const int64_t q_row = r < L ? r : r - L;
                kv_source src = queue_source(k, v, kv_cache, c, h, L, H, D);
                src.window = 1;
                src.map_src = map;
                src.map_chunk = map + max_nk;
                src.map_row = map + 2 * max_nk;
                attend_row(dtype, q, ((q_chunk * L + q_row) * H + h) * D, &src, nk, scale, s,
                           dst, NULL);
            }
        }
        free(s);
        free(map);
    }
    return bad ? -2 : 0;
}

/* ---- streaming queue over a ring of slots ----------------------------- */

/* Slot of the queue's chunk c (processing order, c = 0 the tail). */
int64_t oracle_ring_slot(int64_t slots, int64_t tail_slot, int64_t c)
{
    int64_t p = (tail_slot - c) % slots;
    return p < 0 ? p + slots : p;
}

/*
 * Queue step over the n_live chunks of a ring, selected rows (chunk c in
 * processing order, head, row); out: n_rows x D.  The key/value set of chunk c
 * is [the predecessor's rows (c >= 1)] ++ [its own rows], both read in place
 * from their slots.
 */
int oracle_ring_rows(int dtype, const void *q, const void *k, const void *v, int64_t slots,
                     int64_t tail_slot, int64_t n_live, int64_t L, int64_t H, int64_t D,
                     double scale, const int64_t *rows, int64_t n_rows, double *out)
{
    if (slots <= 0 || n_live <= 0 || n_live > slots || tail_slot < 0 || tail_slot >= slots ||
        L <= 0 || H <= 0 || D <= 0)
        return -1;
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t c = rows[3 * i], h = rows[3 * i + 1], r = rows[3 * i + 2];
        if (c < 0 || c >= n_live || h < 0 || h >= H || r < 0 || r >= L)
            return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * 2 * L);
        int64_t *map = (int64_t *)malloc(sizeof(int64_t) * 3 * 2 * L);
        if (!s || !map) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < n_rows; ++i) {
                const int64_t c = rows[3 * i], h = rows[3 * i + 1], r = rows[3 * i + 2];
                /* R_c as (source, slot, row): predecessor slot, then own slot */
                int64_t nk = 0;
                int64_t *src = map, *slot = map + 2 * L, *row = map + 4 * L;
                if (c >= 1)
                    for (int64_t j = 0; j < L; ++j, ++nk) {
                        src[nk] = ORACLE_SRC_OWN;  /* read in place, not from a cache */
                        slot[nk] = oracle_ring_slot(slots, tail_slot, c - 1);
                        row[nk] = j;
                    }
                for (int64_t j = 0; j < L; ++j, ++nk) {
                    src[nk] = ORACLE_SRC_OWN;
                    slot[nk] = oracle_ring_slot(slots, tail_slot, c);
                    row[nk] = j;
                }
                kv_source ks = queue_source(k, v, NULL, 0, h, L, H, D);
                ks.window = 1;  /* explicit (source, chunk slot, row) list */
                ks.map_src = src;
                ks.map_chunk = slot;
                ks.map_row = row;
                const int64_t q_off =
                    ((oracle_ring_slot(slots, tail_slot, c) * L + r) * H + h) * D;
                attend_row(dtype, q, q_off, &ks, nk, scale, s, out + i * D, NULL);
            }
        }
        free(s);
        free(map);
    }
    return bad ? -2 : 0;
}
