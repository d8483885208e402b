/*
 * pa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU implementation of what the paged-KV decode path computes,
 * in fp64, used to check the GPU library. It shares no code, header, table or
 * constant with the GPU path and must never be linked into it: only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark load it.
 *
 * Sources (cited by short tag below):
 *   [vk]   vaibhawkumar.in, "Why LLMs run out of VRAM: KV cache fragmentation
 *          and the PagedAttention fix"
 *   [devto] dev.to (Syed Anzar), "Why LLMs Run Out of VRAM: KV Cache
 *          Fragmentation and How PagedAttention Fixes It"
 *   [hi]   hyperinfer.ai, "KV cache & paged attention deep dive"
 *   OCP    Open Compute Project, "OCP 8-bit Floating Point Specification
 *          (OFP8)", E4M3 encoding.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes):
 *   - Query head h reads KV head h / (Hq/Hkv) (consecutive grouping of GQA,
 *     [devto] §2 "Example 2").
 *   - Within one physical block and KV head, K is stored token-major
 *     ([bs][D]) and V as bs/16 tiles of 16 consecutive tokens each; bs is a
 *     multiple of 16.  Inside a V tile, with p = 4 / (bytes per element),
 *     the value of token u and dim d is element
 *         ((((d / 16p) * 4 + u / 4) * 16 + d % 16) * p + (d / 16) % p) * 4 + u % 4,
 *     so each 16-byte piece holds p dims (16 apart) of 4 consecutive tokens,
 *     and D is a multiple of 16p.  The pages fix only that a block holds a
 *     fixed number of consecutive tokens ([devto] §4).
 *   - The decoded token attends to every cached token including the one just
 *     appended ([devto] §1: append, then attend over the stored history).
 *   - FP8 is OCP E4M3FN (bias 7, max 448, no infinities); the pages only say
 *     "FP8 (1 byte)" ([devto] §2, §6; [hi] "KV quantization").
 *   - Quantisation multiplies by inv = fl32(1/scale) in fp32, then rounds to
 *     the nearest E4M3 value, ties to the even code, saturating at +-448.
 *   - A sequence of length 0 yields a zero output row.
 *
 * Parity status: every function here is pinned by CPU tests against closed
 * forms, brute force or library routines (see tests/test_oracle_*.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* dtype codes understood by the oracle (its own numbering). */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_E4M3 = 3 };

int orc_elem_bytes(int dtype)
{
    switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_E4M3: return 1;
    default: return 0;
    }
}

/* ---------------------------------------------------------------------- */
/* Number formats, each from its published definition.                    */
/* ---------------------------------------------------------------------- */

/* OCP E4M3: sign s, 4 exponent bits e (bias 7), 3 mantissa bits m.
 * e == 0 is subnormal: (-1)^s * m/8 * 2^(1-7).  S.1111.111 is NaN; every
 * other code with e == 15 is an ordinary normal number (no infinities). */
double orc_e4m3_to_double(uint8_t c)
{
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - 7);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* IEEE 754 binary16: 5 exponent bits (bias 15), 10 mantissa bits. */
double orc_f16_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double mag;
    if (e == 31)
        mag = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)m / 1024.0, -14);
    else
        mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return s ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double orc_f32_to_double(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* The 256 E4M3 values, filled once from the definition above; a table so
 * that long sequences decode in reasonable time. */
static double e4m3_table[256];
static pthread_once_t e4m3_once = PTHREAD_ONCE_INIT;

static void e4m3_fill(void)
{
    for (int c = 0; c < 256; ++c)
        e4m3_table[c] = orc_e4m3_to_double((uint8_t)c);
}

static double e4m3_value(uint8_t c)
{
    pthread_once(&e4m3_once, e4m3_fill);
    return e4m3_table[c];
}

/* Read element `i` of an array of the given dtype as an exact double. */
double orc_load(int dtype, const void *base, size_t i)
{
    const uint8_t *p = (const uint8_t *)base;
    switch (dtype) {
    case ORC_F32: {
        uint32_t u;
        memcpy(&u, p + 4 * i, 4);
        return orc_f32_to_double(u);
    }
    case ORC_F16: {
        uint16_t u;
        memcpy(&u, p + 2 * i, 2);
        return orc_f16_to_double(u);
    }
    case ORC_BF16: {
        uint16_t u;
        memcpy(&u, p + 2 * i, 2);
        return orc_bf16_to_double(u);
    }
    case ORC_E4M3:
        return e4m3_value(p[i]);
    }
    return NAN;
}

/* Encode an fp32 value as E4M3: the nearest finite E4M3 value, a tie going to
 * the code whose last mantissa bit is 0.  Magnitudes at or above the largest
 * finite value (448) saturate to it; NaN maps to the NaN code with the input's
 * sign.  Positive codes 0..126 are in increasing order of value, so the two
 * neighbours of |x| are found by bisection over their values. */
uint8_t orc_e4m3_from_float(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint8_t sign = (u >> 31) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (isnan(x))
        return sign | 0x7F;
    if (a >= 448.0)
        return sign | 0x7E;
    int lo = 0, hi = 0x7E; /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double below = a - e4m3_value((uint8_t)lo);
    double above = e4m3_value((uint8_t)hi) - a;
    int c;
    if (below < above)
        c = lo;
    else if (above < below)
        c = hi;
    else
        c = (lo & 1) == 0 ? lo : hi;
    return sign | (uint8_t)c;
}

/* Sizes from the pages' closed form: bytes per token = 2 x layers x kv_heads
 * x head_dim x bytes per element ([devto] §2 "The Concrete Math of KV Cache
 * Growth"; the same product in [hi] "What the KV cache is"). */
uint64_t orc_kv_bytes_per_token(int64_t layers, int64_t kv_heads, int64_t head_dim,
                                int64_t elem_bytes)
{
    return (uint64_t)(2 * layers * kv_heads * head_dim * elem_bytes);
}

/* ---------------------------------------------------------------------- */
/* Cache append ([devto] §1: the new token's K and V are appended to the   */
/* cache; §4: a token's slot is (physical block, offset inside block)).    */
/* ---------------------------------------------------------------------- */

typedef struct {
    int32_t num_blocks;   /* physical blocks in the pool */
    int32_t block_size;   /* tokens per block */
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t kv_dtype;     /* storage dtype of the cache */
    int32_t in_dtype;     /* dtype of the new tokens' K and V */
} orc_cache_desc;

/* Element index of (blk, g, o, d) in the K cache and in the V cache. */
static size_t k_index(const orc_cache_desc *c, int64_t blk, int g, int o, int d)
{
    return (((size_t)blk * c->num_kv_heads + g) * c->block_size + o) * c->head_dim + d;
}

/* V: tile o / 16 of (blk, g); inside it, token u = o % 16 and dim d sit in
 * 16-byte piece (d / 16p) * 64 + (u / 4) * 16 + d % 16, which holds p dims
 * of 4 tokens, at place ((d / 16) % p) * 4 + u % 4; p = 4 / element bytes. */
static size_t v_index(const orc_cache_desc *c, int64_t blk, int g, int o, int d)
{
    const size_t tile = ((size_t)blk * c->num_kv_heads + g) * (c->block_size / 16) + o / 16;
    const int p = 4 / orc_elem_bytes(c->kv_dtype);
    const int u = o % 16;
    const size_t piece = (size_t)(d / (16 * p)) * 64 + (size_t)(u / 4) * 16 + d % 16;
    return tile * 16 * c->head_dim + piece * 4 * p + (size_t)((d / 16) % p) * 4 + u % 4;
}

/* Store one value of the new token into the cache slot. */
static void store_elem(const orc_cache_desc *c, void *cache, size_t idx, const void *src,
                       size_t src_idx, float scale)
{
    uint8_t *dst = (uint8_t *)cache;
    const uint8_t *s = (const uint8_t *)src;
    if (c->kv_dtype == c->in_dtype) {
        int eb = orc_elem_bytes(c->kv_dtype);
        memcpy(dst + idx * eb, s + src_idx * eb, eb);
        return;
    }
    /* The only conversion on the path: 16-bit activations into E4M3. */
    float x = (float)orc_load(c->in_dtype, src, src_idx); /* exact */
    float inv = 1.0f / scale;
    float y = x * inv; /* one fp32 rounding, as the reading states */
    dst[idx] = orc_e4m3_from_float(y);
}

typedef struct {
    const orc_cache_desc *c;
    const void *k_new, *v_new;
    void *k_cache, *v_cache;
    const int32_t *slots;
    int32_t t0, t1;
    float k_scale, v_scale;
} append_job;

/* Writes tokens [t0, t1) of one job; slots were checked by the caller. */
static void *append_worker(void *arg)
{
    const append_job *J = (const append_job *)arg;
    const orc_cache_desc *c = J->c;
    for (int32_t t = J->t0; t < J->t1; ++t) {
        int64_t slot = J->slots[t];
        if (slot < 0)
            continue;
        int64_t blk = slot / c->block_size;
        int o = (int)(slot % c->block_size);
        for (int g = 0; g < c->num_kv_heads; ++g) {
            for (int d = 0; d < c->head_dim; ++d) {
                size_t src = ((size_t)t * c->num_kv_heads + g) * c->head_dim + d;
                store_elem(c, J->k_cache, k_index(c, blk, g, o, d), J->k_new, src, J->k_scale);
                store_elem(c, J->v_cache, v_index(c, blk, g, o, d), J->v_new, src, J->v_scale);
            }
        }
    }
    return NULL;
}

/* k_new, v_new: [num_tokens][Hkv][D] in in_dtype.  slot_mapping[t] is
 * block * block_size + offset, or negative to skip the token.  Tokens are
 * independent (their slots are distinct), so ranges of them are written by
 * separate threads.  Returns 0, or -1 if a slot lies outside the pool, the
 * dtype pair is not one the path defines, block_size is not a positive
 * multiple of 16 or head_dim not one of 16 p (p = 4 / element bytes). */
int orc_cache_append(const orc_cache_desc *c, const void *k_new, const void *v_new,
                     void *k_cache, void *v_cache, const int32_t *slot_mapping,
                     int32_t num_tokens, float k_scale, float v_scale)
{
    if (!(c->kv_dtype == c->in_dtype ||
          (c->kv_dtype == ORC_E4M3 && (c->in_dtype == ORC_BF16 || c->in_dtype == ORC_F16))) ||
        c->block_size <= 0 || c->block_size % 16 != 0 || c->head_dim <= 0 ||
        c->head_dim % (64 / orc_elem_bytes(c->kv_dtype)) != 0)
        return -1;
    for (int32_t t = 0; t < num_tokens; ++t)
        if (slot_mapping[t] >= (int64_t)c->num_blocks * c->block_size)
            return -1;
    int nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 64)
        nthreads = 64;
    if (num_tokens < 1024)
        nthreads = 1;
    append_job jobs[64];
    pthread_t th[64];
    int started[64] = {0};
    for (int i = 0; i < nthreads; ++i) {
        append_job j = {c, k_new, v_new, k_cache, v_cache, slot_mapping,
                        (int32_t)((int64_t)num_tokens * i / nthreads),
                        (int32_t)((int64_t)num_tokens * (i + 1) / nthreads), k_scale, v_scale};
        jobs[i] = j;
    }
    for (int i = 1; i < nthreads; ++i)
        started[i] = pthread_create(&th[i], NULL, append_worker, &jobs[i]) == 0;
    append_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (started[i])
            pthread_join(th[i], NULL);
        else
            append_worker(&jobs[i]);
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Decode: single-query attention over the tokens a block table gathers.   */
/*   out = softmax(q K^T * scale) V          ([devto] §1, attention eq.)    */
/*   token t of sequence b lives in physical block table[b][t / bs] at      */
/*   offset t % bs                           ([devto] §4, block table)      */
/*   With a window start w (optional), only tokens w..n-1 take part: the    */
/*   sliding window keeps the most recent tokens; the earlier ones of the   */
/*   first kept block stay stored but are left out ([vk] "PagedAttention:   */
/*   the idea" and its truncate sketch).  w = n gives a zero row.           */
/* ---------------------------------------------------------------------- */

typedef struct {
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
    int32_t max_blocks_per_seq; /* row stride of block_tables */
    int32_t q_dtype;
    int32_t kv_dtype;
} orc_decode_desc;

typedef struct {
    const orc_decode_desc *d;
    const void *q, *k_cache, *v_cache;
    const int32_t *block_tables, *seq_lens, *seq_starts;
    double scale, k_scale, v_scale;
    const int32_t *rows; /* NULL: all rows b*Hq+h; else list of row ids */
    int64_t num_rows;
    double *out; /* [num_rows][D] */
    int64_t next;
    pthread_mutex_t lock;
    int status;
} decode_job;

/* One output row (b, h).  Two passes over the tokens: scores, then the
 * normalised weighted sum of V, exactly as the formula reads. */
static int decode_row(const decode_job *J, int64_t row, double *out_row, double *s)
{
    const orc_decode_desc *d = J->d;
    int G = d->num_q_heads / d->num_kv_heads;
    int b = (int)(row / d->num_q_heads);
    int h = (int)(row % d->num_q_heads);
    int g = h / G;
    int D = d->head_dim;
    int64_t n = J->seq_lens[b];
    int64_t w = J->seq_starts ? J->seq_starts[b] : 0; /* first token of the window */
    orc_cache_desc c = {d->num_blocks, d->block_size, d->num_kv_heads, D, d->kv_dtype,
                        d->q_dtype};

    for (int i = 0; i < D; ++i)
        out_row[i] = 0.0;
    if (n < 0 || n > (int64_t)d->max_blocks_per_seq * d->block_size || w < 0 || w > n)
        return -1;
    if (w == n)
        return 0;

    const int32_t *table = J->block_tables + (size_t)b * d->max_blocks_per_seq;
    size_t qbase = ((size_t)b * d->num_q_heads + h) * D;
    double qv[1024];
    if (D > 1024)
        return -3;
    for (int i = 0; i < D; ++i)
        qv[i] = orc_load(d->q_dtype, J->q, qbase + i);

    /* scores s_t = scale * sum_d q[d] * (k_scale * K_t[d]) */
    for (int64_t t = w; t < n; ++t) {
        int64_t blk = table[t / d->block_size];
        int o = (int)(t % d->block_size);
        if (blk < 0 || blk >= d->num_blocks)
            return -1;
        double dot = 0.0;
        for (int i = 0; i < D; ++i) {
            double ki = orc_load(d->kv_dtype, J->k_cache, k_index(&c, blk, g, o, i)) * J->k_scale;
            dot += qv[i] * ki;
        }
        s[t] = J->scale * dot;
    }
    /* softmax weights w_t = exp(s_t - max s) / sum */
    double m = -INFINITY;
    for (int64_t t = w; t < n; ++t)
        if (s[t] > m)
            m = s[t];
    double Z = 0.0;
    for (int64_t t = w; t < n; ++t) {
        s[t] = exp(s[t] - m);
        Z += s[t];
    }
    /* out = sum_t w_t * (v_scale * V_t) / Z */
    for (int64_t t = w; t < n; ++t) {
        int64_t blk = table[t / d->block_size];
        int o = (int)(t % d->block_size);
        for (int i = 0; i < D; ++i) {
            double vi = orc_load(d->kv_dtype, J->v_cache, v_index(&c, blk, g, o, i)) * J->v_scale;
            out_row[i] += s[t] * vi;
        }
    }
    for (int i = 0; i < D; ++i)
        out_row[i] /= Z;
    return 0;
}

static void *decode_worker(void *arg)
{
    decode_job *J = (decode_job *)arg;
    int64_t max_n = (int64_t)J->d->max_blocks_per_seq * J->d->block_size;
    double *s = (double *)malloc(sizeof(double) * (size_t)(max_n > 0 ? max_n : 1));
    if (!s) {
        pthread_mutex_lock(&J->lock);
        J->status = -2;
        pthread_mutex_unlock(&J->lock);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t i = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (i >= J->num_rows)
            break;
        int64_t row = J->rows ? J->rows[i] : i;
        int rc = decode_row(J, row, J->out + (size_t)i * J->d->head_dim, s);
        if (rc) {
            pthread_mutex_lock(&J->lock);
            J->status = rc;
            pthread_mutex_unlock(&J->lock);
        }
    }
    free(s);
    return NULL;
}

/* q: [B][Hq][D] in q_dtype; caches as described above; block_tables:
 * [B][max_blocks_per_seq]; seq_lens: [B]; seq_starts: [B] window starts, or
 * NULL for windows that start at token 0.  rows: optional list of row ids
 * (b * Hq + h) to compute, or NULL for all B*Hq rows; out: [rows][D] fp64.
 * nthreads <= 0 uses every online CPU.  Returns 0, or -1 on a bad table
 * entry / length, -2 on allocation failure, -3 on a bad shape. */
int orc_decode(const orc_decode_desc *d, const void *q, const void *k_cache,
               const void *v_cache, const int32_t *block_tables, const int32_t *seq_lens,
               const int32_t *seq_starts, double scale, double k_scale, double v_scale,
               const int32_t *rows,
               int64_t num_rows, double *out, int nthreads)
{
    if (d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0 || d->head_dim <= 0 ||
        d->block_size <= 0 || d->block_size % 16 != 0 ||
        d->head_dim % (64 / orc_elem_bytes(d->kv_dtype)) != 0)
        return -3;
    decode_job J;
    J.d = d;
    J.q = q;
    J.k_cache = k_cache;
    J.v_cache = v_cache;
    J.block_tables = block_tables;
    J.seq_lens = seq_lens;
    J.seq_starts = seq_starts;
    J.scale = scale;
    J.k_scale = k_scale;
    J.v_scale = v_scale;
    J.rows = rows;
    J.num_rows = rows ? num_rows : (int64_t)d->num_seqs * d->num_q_heads;
    J.out = out;
    J.next = 0;
    J.status = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads <= 0)
        nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, decode_worker, &J) == 0)
            ++started;
    decode_worker(&J);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.lock);
    return J.status;
}
