/*
 * fd_oracle.c -- TEST INFRASTRUCTURE.  A plain, slow float64 CPU reference for
 * decode attention with the unified-max split-KV softmax.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg load it; the GPU library
 * never does, and the two share no source.
 *
 * What is computed (FlashDecoding++ theory page, section 1: a length-1 query
 * scored against a KV cache that keeps growing; section 3: the softmax and the
 * safe-band fallback):
 *
 *   s_t   = scale * sum_d q_d * k_{t,d}                (k dequantised: code * k_scale)
 *   out   = sum_t exp(s_t - max_j s_j) v_t / sum_t exp(s_t - max_j s_j)
 *   flag  = 1 if any valid s_t lies outside [phi - a, phi + b]   (closed band)
 *
 * orc_decode_exact() is that plain definition: the method reaches exactly this
 * result up to rounding order, because exp(x - phi)/sum exp(x - phi) equals the
 * max-subtracted softmax (theory page, section 3, both displayed formulas) and
 * flagged rows are recomputed exactly.
 *
 * orc_decode_unified() walks the method's own steps in the page's order, in
 * float64: per chunk the sums exp(s - phi) and exp(s - phi) v against the
 * preset constant; a chunk with a score outside the band is recomputed with
 * the running-max online softmax; chunks are merged by a plain sum (with the
 * ordinary max rescale only when a chunk was recomputed).  Tests use it to show
 * that the unified form equals the exact one and does not depend on the chunk
 * count.
 *
 * Storage formats decoded here, each from its definition:
 *   f32   -- IEEE binary32
 *   bf16  -- upper 16 bits of a binary32
 *   E4M3FN (OCP 8-bit float) -- sign, 4 exponent bits (bias 7), 3 mantissa
 *            bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is
 *            NaN; no infinities.  Real value = k_scale * decoded code
 *            (symmetric scale, as the quantisation background page defines it).
 *
 * Layouts:
 *   q, out       [B][Hq][D]
 *   contiguous K/V [B][Hkv][max_seq_len][D]
 *   paged K/V    [num_pages][Hkv][page_size][D]; token t of sequence b lives in
 *                page block_table[b][t / page_size] at slot t % page_size
 *   query head h reads KV head h / (Hq / Hkv)
 *
 * The prefill form (a causal block of queries per sequence, same unified
 * maximum and band) and the calibration statistics (choosing phi and the
 * band from observed scores) have sections of their own at the end.
 *
 * Readings taken where the pages are silent: the band is closed at both ends
 * and a NaN score is outside it; tokens t >= seq_lens[b] are not attended and
 * not tested; a sequence of length <= 0 gives a zero row with flag 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3FN = 2 };

typedef struct {
    int32_t batch, num_q_heads, num_kv_heads, head_dim;
    int32_t max_seq_len;          /* contiguous capacity; also clamps seq_lens */
    int32_t page_size;            /* 0 = contiguous */
    int32_t max_blocks_per_seq;   /* row stride of block_table */
    int32_t q_dtype, kv_dtype;
    double scale;
} orc_problem;

typedef struct {
    const void *q, *k, *v;
    const int32_t *seq_lens, *block_table;
    const float *k_scale, *v_scale;
} orc_inputs;

/* ---------------------------------------------------------------- decoding */

double orc_decode_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double orc_decode_e4m3fn(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);                 /* (m/8) * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

static double elem(const void *base, size_t i, int dtype)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[i];
    case ORC_BF16: return orc_decode_bf16(((const uint16_t *)base)[i]);
    default: return orc_decode_e4m3fn(((const uint8_t *)base)[i]);
    }
}

/* element offset of (sequence b, kv head kvh, token t, component 0) */
static size_t kv_offset(const orc_problem *p, const int32_t *block_table, int b, int kvh, int t)
{
    if (p->page_size == 0)
        return (((size_t)b * p->num_kv_heads + kvh) * p->max_seq_len + t) * p->head_dim;
    int32_t page = block_table[(size_t)b * p->max_blocks_per_seq + t / p->page_size];
    return (((size_t)page * p->num_kv_heads + kvh) * p->page_size + t % p->page_size)
           * p->head_dim;
}

static int seq_len_of(const orc_problem *p, const orc_inputs *in, int b)
{
    int L = in->seq_lens[b];
    if (L < 0) L = 0;
    if (L > p->max_seq_len) L = p->max_seq_len;
    return L;
}

/* all scores of row (b, h): s_t = scale * sum_d q_d k_{t,d}, t < L */
static void row_scores(const orc_problem *p, const orc_inputs *in, int b, int h, int L, double *s)
{
    const int D = p->head_dim;
    const int kvh = h / (p->num_q_heads / p->num_kv_heads);
    const double ks = (p->kv_dtype == ORC_E4M3FN) ? (double)in->k_scale[kvh] : 1.0;
    double *qd = malloc(sizeof(double) * D);
    for (int d = 0; d < D; d++)
        qd[d] = elem(in->q, ((size_t)b * p->num_q_heads + h) * D + d, p->q_dtype);
    for (int t = 0; t < L; t++) {
        size_t off = kv_offset(p, in->block_table, b, kvh, t);
        double acc = 0.0;
        for (int d = 0; d < D; d++)
            acc += qd[d] * (ks * elem(in->k, off + d, p->kv_dtype));
        s[t] = p->scale * acc;
    }
    free(qd);
}

/* acc[d] = acc[d] * r + w * v_{t,d}   (v dequantised: code * v_scale) */
static void accumulate_value(const orc_problem *p, const orc_inputs *in, int b, int kvh, int t,
                             double r, double w, double *acc)
{
    const double vs = (p->kv_dtype == ORC_E4M3FN) ? (double)in->v_scale[kvh] : 1.0;
    const size_t off = kv_offset(p, in->block_table, b, kvh, t);
    for (int d = 0; d < p->head_dim; d++)
        acc[d] = acc[d] * r + w * (vs * elem(in->v, off + d, p->kv_dtype));
}

static int outside_band(double s, double lo, double hi)
{
    return !(s >= lo && s <= hi);
}

/* ------------------------------------------------------------ exact softmax */

static void exact_row(const orc_problem *p, const orc_inputs *in, int row, double phi,
                      double a, double b_, double *out, uint8_t *flag, double *margin)
{
    const int D = p->head_dim;
    const int b = row / p->num_q_heads, h = row % p->num_q_heads;
    const int kvh = h / (p->num_q_heads / p->num_kv_heads);
    const int L = seq_len_of(p, in, b);
    const double lo = phi - a, hi = phi + b_;

    for (int d = 0; d < D; d++) out[d] = 0.0;
    *flag = 0;
    if (margin) *margin = INFINITY;
    if (L == 0) return;

    double *s = malloc(sizeof(double) * L);
    row_scores(p, in, b, h, L, s);

    int has_nan = 0;
    double m = -INFINITY, mg = INFINITY;
    for (int t = 0; t < L; t++) {
        if (outside_band(s[t], lo, hi)) *flag = 1;
        if (isnan(s[t])) has_nan = 1;
        else if (s[t] > m) m = s[t];
        double dist = fmin(fabs(s[t] - lo), fabs(s[t] - hi));
        if (!(dist >= mg)) mg = dist;
    }
    if (margin) *margin = mg;

    if (has_nan) {
        for (int d = 0; d < D; d++) out[d] = NAN;
        free(s);
        return;
    }
    double l = 0.0;
    for (int t = 0; t < L; t++) {
        double w = exp(s[t] - m);
        l += w;
        accumulate_value(p, in, b, kvh, t, 1.0, w, out);
    }
    for (int d = 0; d < D; d++) out[d] /= l;
    free(s);
}

/*
 * Caps the OpenMP threads of the calls that follow at n (n < 1: back to the
 * runtime's default).  Used to time the oracle on one core beside all cores.
 */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    static int dflt = 0;
    if (dflt == 0) dflt = omp_get_max_threads();
    omp_set_num_threads(n > 0 ? n : dflt);
#else
    (void)n;
#endif
}

/*
 * rows: nrows row ids (b * Hq + h), or NULL for all B*Hq rows in order.
 * out: [nrows][D]; flags: [nrows]; margin: [nrows] or NULL -- the smallest
 * distance from any valid score to either band edge (infinity for empty rows).
 * Returns the number of threads used.
 */
int orc_decode_exact(const orc_problem *p, const orc_inputs *in, double phi, double a, double b,
                     int nrows, const int32_t *rows, double *out, uint8_t *flags, double *margin)
{
    int threads = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        threads = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < nrows; i++) {
            int row = rows ? rows[i] : i;
            exact_row(p, in, row, phi, a, b, out + (size_t)i * p->head_dim, flags + i,
                      margin ? margin + i : NULL);
        }
    }
    return threads;
}

/* scores of one row (b, h), float64, s[0 .. seq_len) ; returns the length */
int orc_scores(const orc_problem *p, const orc_inputs *in, int b, int h, double *s)
{
    int L = seq_len_of(p, in, b);
    row_scores(p, in, b, h, L, s);
    return L;
}

/* ------------------------------------------- the method's steps, in float64 */

static void unified_row(const orc_problem *p, const orc_inputs *in, int row, int chunk,
                        double phi, double a, double b_, double *out, uint8_t *flag,
                        int32_t *recomputed)
{
    const int D = p->head_dim;
    const int b = row / p->num_q_heads, h = row % p->num_q_heads;
    const int kvh = h / (p->num_q_heads / p->num_kv_heads);
    const int L = seq_len_of(p, in, b);
    const double lo = phi - a, hi = phi + b_;
    const int nch = (L + chunk - 1) / chunk;

    for (int d = 0; d < D; d++) out[d] = 0.0;
    *flag = 0;
    *recomputed = 0;
    if (L == 0) return;

    double *s = malloc(sizeof(double) * L);
    row_scores(p, in, b, h, L, s);
    double *m_c = malloc(sizeof(double) * nch);
    double *l_c = malloc(sizeof(double) * nch);
    double *o_c = calloc((size_t)nch * D, sizeof(double));
    uint8_t *bad = calloc(nch, 1);

    for (int c = 0; c < nch; c++) {
        const int t0 = c * chunk, t1 = (t0 + chunk < L) ? t0 + chunk : L;
        double *o = o_c + (size_t)c * D;
        /* asynchronous partial against the preset constant phi */
        l_c[c] = 0.0;
        m_c[c] = phi;
        for (int t = t0; t < t1; t++) {
            if (outside_band(s[t], lo, hi)) bad[c] = 1;
            double w = exp(s[t] - phi);
            l_c[c] += w;
            accumulate_value(p, in, b, kvh, t, 1.0, w, o);
        }
        if (!bad[c]) continue;
        /* this chunk left the band: discard it, redo it with online softmax */
        *flag = 1;
        (*recomputed)++;
        double m = -INFINITY, l = 0.0;
        for (int d = 0; d < D; d++) o[d] = 0.0;
        for (int t = t0; t < t1; t++) {
            double m_new = (s[t] > m || isnan(s[t])) ? s[t] : m;
            double r = exp(m - m_new);       /* rescale of what was accumulated */
            double w = (s[t] == -INFINITY) ? 0.0 : exp(s[t] - m_new);
            if (m == -INFINITY) r = 0.0;     /* nothing accumulated yet */
            l = l * r + w;
            accumulate_value(p, in, b, kvh, t, r, w, o);
            m = m_new;
        }
        m_c[c] = m;
        l_c[c] = l;
    }

    double M = phi;
    if (*flag) {                       /* ordinary max-rescaled merge */
        M = -INFINITY;
        for (int c = 0; c < nch; c++)
            if (isnan(m_c[c]) || m_c[c] > M) M = m_c[c];
    }
    double l = 0.0;
    for (int c = 0; c < nch; c++) {
        /* plain sum when no chunk was recomputed: every m_c equals phi */
        double f = *flag ? exp(m_c[c] - M) : 1.0;
        l += f * l_c[c];
        for (int d = 0; d < D; d++) out[d] += f * o_c[(size_t)c * D + d];
    }
    for (int d = 0; d < D; d++) out[d] /= l;

    free(s); free(m_c); free(l_c); free(o_c); free(bad);
}

int orc_decode_unified(const orc_problem *p, const orc_inputs *in, int chunk, double phi,
                       double a, double b, int nrows, const int32_t *rows, double *out,
                       uint8_t *flags, int32_t *recomputed)
{
    int threads = 1;
    if (chunk <= 0) return -1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        threads = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < nrows; i++) {
            int row = rows ? rows[i] : i;
            unified_row(p, in, row, chunk, phi, a, b, out + (size_t)i * p->head_dim, flags + i,
                        recomputed + i);
        }
    }
    return threads;
}

/* ------------------------------------------------------------------ prefill */
/*
 * Prefill: a block of Lq query tokens per sequence attends causally to the
 * sequence's keys (FlashDecoding++ theory page, section 3: the same unified
 * maximum serves the prefill phase; section 1: prefill processes all prompt
 * tokens at once).  Layouts and reading:
 *
 *   q, out   [B][Hq][Lq][D]      flags [B][Hq][Lq]
 *   K/V      contiguous [B][Hkv][max_seq_len][D], or paged
 *            [pages][Hkv][page_size][D] with token t of sequence b in page
 *            block_table[b][t / page_size], slot t % page_size (the decode
 *            cache layouts); E4M3FN codes times the per-KV-head k_scale /
 *            v_scale (the symmetric scale of the quantisation page)
 *   query j of sequence b sits at position pos = kv_lens[b] - Lq + j
 *   (kv_lens clamped to [0, max_seq_len]) and attends keys t = 0 .. pos;
 *   a query with pos < 0 has no key: zero row, flag 0.
 *
 * orc_prefill_exact() is the plain definition (max-subtracted softmax over
 * the visible keys, plus the band test over those scores).
 * orc_prefill_unified() follows the method: key tiles of `tile` tokens, each
 * reduced against the preset phi; a tile with a visible score outside the
 * band is redone with online softmax; tiles merged by a plain sum (max
 * rescale only when a tile was redone).
 */
typedef struct {
    int32_t batch, num_q_heads, num_kv_heads, head_dim;
    int32_t max_seq_len, q_len;
    int32_t q_dtype, kv_dtype;       /* q: ORC_F32 or ORC_BF16; K/V: also ORC_E4M3FN */
    int32_t page_size;               /* 0 = contiguous */
    int32_t max_blocks_per_seq;      /* row stride of block_table */
    double scale;
} orc_prefill_problem;

typedef struct {
    const void *q, *k, *v;
    const int32_t *kv_lens, *block_table;
    const float *k_scale, *v_scale;  /* [Hkv], E4M3FN only */
} orc_prefill_inputs;

/* element offset of (sequence b, kv head kvh, key t, component 0) */
static size_t prefill_kv_offset(const orc_prefill_problem *p, const orc_prefill_inputs *in, int b, int kvh,
                                int t)
{
    if (p->page_size == 0)
        return (((size_t)b * p->num_kv_heads + kvh) * p->max_seq_len + t) * p->head_dim;
    int32_t page = in->block_table[(size_t)b * p->max_blocks_per_seq + t / p->page_size];
    return (((size_t)page * p->num_kv_heads + kvh) * p->page_size + t % p->page_size) * p->head_dim;
}

/* keys visible to query j of sequence b */
static int prefill_keys(const orc_prefill_problem *p, const orc_prefill_inputs *in, int b, int j)
{
    int kv = in->kv_lens[b];
    if (kv < 0) kv = 0;
    if (kv > p->max_seq_len) kv = p->max_seq_len;
    int pos = kv - p->q_len + j;
    return pos < 0 ? 0 : pos + 1;
}

/* scores of query row (b, h, j) against keys 0 .. n-1 */
static void prefill_scores(const orc_prefill_problem *p, const orc_prefill_inputs *in, int b, int h,
                           int j, int n, double *s)
{
    const int D = p->head_dim;
    const int kvh = h / (p->num_q_heads / p->num_kv_heads);
    const double ks = (p->kv_dtype == ORC_E4M3FN) ? (double)in->k_scale[kvh] : 1.0;
    double *qd = malloc(sizeof(double) * D);
    for (int d = 0; d < D; d++)
        qd[d] = elem(in->q, (((size_t)b * p->num_q_heads + h) * p->q_len + j) * D + d, p->q_dtype);
    for (int t = 0; t < n; t++) {
        size_t off = prefill_kv_offset(p, in, b, kvh, t);
        double acc = 0.0;
        for (int d = 0; d < D; d++) acc += qd[d] * (ks * elem(in->k, off + d, p->kv_dtype));
        s[t] = p->scale * acc;
    }
    free(qd);
}

static void prefill_value(const orc_prefill_problem *p, const orc_prefill_inputs *in, int b, int kvh,
                          int t, double r, double w, double *acc)
{
    const size_t off = prefill_kv_offset(p, in, b, kvh, t);
    const double vs = (p->kv_dtype == ORC_E4M3FN) ? (double)in->v_scale[kvh] : 1.0;
    for (int d = 0; d < p->head_dim; d++)
        acc[d] = acc[d] * r + w * (vs * elem(in->v, off + d, p->kv_dtype));
}

/* row = (b * Hq + h) * Lq + j */
static void prefill_exact_row(const orc_prefill_problem *p, const orc_prefill_inputs *in, int row,
                              double phi, double a, double b_, double *out, uint8_t *flag,
                              double *margin)
{
    const int D = p->head_dim, Lq = p->q_len;
    const int j = row % Lq, bh = row / Lq;
    const int b = bh / p->num_q_heads, h = bh % p->num_q_heads;
    const int kvh = h / (p->num_q_heads / p->num_kv_heads);
    const int n = prefill_keys(p, in, b, j);
    const double lo = phi - a, hi = phi + b_;

    for (int d = 0; d < D; d++) out[d] = 0.0;
    *flag = 0;
    if (margin) *margin = INFINITY;
    if (n == 0) return;

    double *s = malloc(sizeof(double) * n);
    prefill_scores(p, in, b, h, j, n, s);
    int has_nan = 0;
    double m = -INFINITY, mg = INFINITY;
    for (int t = 0; t < n; t++) {
        if (outside_band(s[t], lo, hi)) *flag = 1;
        if (isnan(s[t])) has_nan = 1;
        else if (s[t] > m) m = s[t];
        double dist = fmin(fabs(s[t] - lo), fabs(s[t] - hi));
        if (!(dist >= mg)) mg = dist;
    }
    if (margin) *margin = mg;
    if (has_nan) {
        for (int d = 0; d < D; d++) out[d] = NAN;
        free(s);
        return;
    }
    double l = 0.0;
    for (int t = 0; t < n; t++) {
        double w = exp(s[t] - m);
        l += w;
        prefill_value(p, in, b, kvh, t, 1.0, w, out);
    }
    for (int d = 0; d < D; d++) out[d] /= l;
    free(s);
}

/* rows: nrows row ids ((b * Hq + h) * Lq + j), or NULL for all in order */
int orc_prefill_exact(const orc_prefill_problem *p, const orc_prefill_inputs *in, double phi,
                      double a, double b, int nrows, const int32_t *rows, double *out,
                      uint8_t *flags, double *margin)
{
    int threads = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        threads = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 4)
        for (int i = 0; i < nrows; i++) {
            int row = rows ? rows[i] : i;
            prefill_exact_row(p, in, row, phi, a, b, out + (size_t)i * p->head_dim, flags + i,
                              margin ? margin + i : NULL);
        }
    }
    return threads;
}

static void prefill_unified_row(const orc_prefill_problem *p, const orc_prefill_inputs *in, int row,
                                int tile, double phi, double a, double b_, double *out,
                                uint8_t *flag, int32_t *redone)
{
    const int D = p->head_dim, Lq = p->q_len;
    const int j = row % Lq, bh = row / Lq;
    const int b = bh / p->num_q_heads, h = bh % p->num_q_heads;
    const int kvh = h / (p->num_q_heads / p->num_kv_heads);
    const int n = prefill_keys(p, in, b, j);
    const double lo = phi - a, hi = phi + b_;
    const int ntile = (n + tile - 1) / tile;

    for (int d = 0; d < D; d++) out[d] = 0.0;
    *flag = 0;
    *redone = 0;
    if (n == 0) return;

    double *s = malloc(sizeof(double) * n);
    prefill_scores(p, in, b, h, j, n, s);
    double *m_c = malloc(sizeof(double) * ntile);
    double *l_c = malloc(sizeof(double) * ntile);
    double *o_c = calloc((size_t)ntile * D, sizeof(double));

    for (int c = 0; c < ntile; c++) {
        const int t0 = c * tile, t1 = (t0 + tile < n) ? t0 + tile : n;
        double *o = o_c + (size_t)c * D;
        int bad = 0;
        l_c[c] = 0.0;
        m_c[c] = phi;
        for (int t = t0; t < t1; t++) {          /* against the preset constant */
            if (outside_band(s[t], lo, hi)) bad = 1;
            double w = exp(s[t] - phi);
            l_c[c] += w;
            prefill_value(p, in, b, kvh, t, 1.0, w, o);
        }
        if (!bad) continue;
        *flag = 1;                               /* redo this tile, online softmax */
        (*redone)++;
        double m = -INFINITY, l = 0.0;
        for (int d = 0; d < D; d++) o[d] = 0.0;
        for (int t = t0; t < t1; t++) {
            double m_new = (s[t] > m || isnan(s[t])) ? s[t] : m;
            double r = (m == -INFINITY) ? 0.0 : exp(m - m_new);
            double w = (s[t] == -INFINITY) ? 0.0 : exp(s[t] - m_new);
            l = l * r + w;
            prefill_value(p, in, b, kvh, t, r, w, o);
            m = m_new;
        }
        m_c[c] = m;
        l_c[c] = l;
    }
    double M = phi;
    if (*flag) {
        M = -INFINITY;
        for (int c = 0; c < ntile; c++)
            if (isnan(m_c[c]) || m_c[c] > M) M = m_c[c];
    }
    double l = 0.0;
    for (int c = 0; c < ntile; c++) {
        double f = *flag ? exp(m_c[c] - M) : 1.0;
        l += f * l_c[c];
        for (int d = 0; d < D; d++) out[d] += f * o_c[(size_t)c * D + d];
    }
    for (int d = 0; d < D; d++) out[d] /= l;
    free(s); free(m_c); free(l_c); free(o_c);
}

int orc_prefill_unified(const orc_prefill_problem *p, const orc_prefill_inputs *in, int tile,
                        double phi, double a, double b, int nrows, const int32_t *rows, double *out,
                        uint8_t *flags, int32_t *redone)
{
    int threads = 1;
    if (tile <= 0) return -1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        threads = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 4)
        for (int i = 0; i < nrows; i++) {
            int row = rows ? rows[i] : i;
            prefill_unified_row(p, in, row, tile, phi, a, b, out + (size_t)i * p->head_dim,
                                flags + i, redone + i);
        }
    }
    return threads;
}

/* -------------------------------------------------------------- calibration */
/*
 * Choosing phi from observed scores (FlashDecoding++ theory page, section 3:
 * phi is set beforehand from the observed score distribution; rows that
 * leave the band take the fallback).
 *
 * orc_score_stats(): per row (b, h) the largest and smallest valid score
 * (empty rows: -inf / +inf) and, when nbins > 0, a histogram of every valid
 * score: counts[0] below lo, counts[1 + i] in [lo + i w, lo + (i+1) w),
 * counts[nbins + 1] at or above hi, w = (hi - lo) / nbins, bins by
 * floor((s - lo) / w) in float64.
 *
 * A row with extremes [mn, mx] stays in band [phi - a, phi + b] iff
 * phi - a <= mn and mx <= phi + b.  A set of rows fits one band of width
 * W = a + b (phi placed anywhere) iff max(mx) - min(mn) <= W over the set.
 * orc_min_band_width(): the smallest W for which all but `allowed` of the
 * non-empty rows fit, by brute force over the smallest minimum of the set.
 * orc_rows_in_band(): how many non-empty rows a given (phi, a, b) keeps.
 */
int orc_score_stats(const orc_problem *p, const orc_inputs *in, double lo, double hi, int nbins,
                    double *row_max, double *row_min, int64_t *counts)
{
    const int rows = p->batch * p->num_q_heads;
    int threads = 1;
    if (nbins > 0) memset(counts, 0, sizeof(int64_t) * (size_t)(nbins + 2));
    const double w = nbins > 0 ? (hi - lo) / nbins : 1.0;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        threads = omp_get_num_threads();
#endif
        double *s = malloc(sizeof(double) * (size_t)(p->max_seq_len > 0 ? p->max_seq_len : 1));
        int64_t *local = nbins > 0 ? calloc((size_t)(nbins + 2), sizeof(int64_t)) : NULL;
#pragma omp for schedule(dynamic, 4)
        for (int r = 0; r < rows; r++) {
            const int b = r / p->num_q_heads, h = r % p->num_q_heads;
            const int n = seq_len_of(p, in, b);
            row_scores(p, in, b, h, n, s);
            double mx = -INFINITY, mn = INFINITY;
            for (int t = 0; t < n; t++) {
                if (s[t] > mx) mx = s[t];
                if (s[t] < mn) mn = s[t];
                if (local) {
                    if (s[t] < lo) local[0]++;
                    else if (s[t] >= hi) local[nbins + 1]++;
                    else {
                        int i = (int)floor((s[t] - lo) / w);
                        if (i >= nbins) i = nbins - 1;   /* rounding right below hi */
                        local[1 + i]++;
                    }
                }
            }
            row_max[r] = mx;
            row_min[r] = mn;
        }
        if (local) {
#pragma omp critical
            for (int i = 0; i < nbins + 2; i++) counts[i] += local[i];
            free(local);
        }
        free(s);
    }
    return threads;
}

int64_t orc_rows_in_band(const double *row_max, const double *row_min, int64_t n, double phi,
                         double a, double b)
{
    int64_t k = 0;
    for (int64_t r = 0; r < n; r++)
        if (row_max[r] >= row_min[r] && phi - a <= row_min[r] && row_max[r] <= phi + b) k++;
    return k;
}

static int cmp_double(const void *x, const void *y)
{
    const double u = *(const double *)x, v = *(const double *)y;
    return (u > v) - (u < v);
}

double orc_min_band_width(const double *row_max, const double *row_min, int64_t n, int64_t allowed)
{
    int64_t m = 0;
    for (int64_t r = 0; r < n; r++)
        if (row_max[r] >= row_min[r]) m++;
    const int64_t need = m - (allowed < 0 ? 0 : allowed);
    if (need <= 0) return 0.0;
    double best = INFINITY;
    double *maxes = malloc(sizeof(double) * (size_t)m);
    for (int64_t j = 0; j < n; j++) {
        if (!(row_max[j] >= row_min[j])) continue;
        const double L = row_min[j];               /* the set's smallest minimum */
        int64_t c = 0;
        for (int64_t r = 0; r < n; r++)
            if (row_max[r] >= row_min[r] && row_min[r] >= L) maxes[c++] = row_max[r];
        if (c < need) continue;
        qsort(maxes, (size_t)c, sizeof(double), cmp_double);
        const double W = maxes[need - 1] - L;
        if (W < best) best = W;
    }
    free(maxes);
    return best;
}
