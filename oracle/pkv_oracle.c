/*
 * pkv_oracle.c -- CPU oracle for paged-KV-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition of what the GPU library computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant with the HIP library, and the library never loads
 * it.  Everything is computed in IEEE double, except the single fp32 division
 * that decides an fp8 code (the same precision the GPU quantiser uses).
 *
 * Sources (web pages about vLLM / PagedAttention):
 *  - bytelighting wiki entry "vLLM", paragraph "Flattened 布局与 slot_mapping":
 *    cu_seqlens (cumulative sequence lengths) keep the requests of a
 *    flattened batch apart; ai-maas.com page, section 引擎的分层结构 (chunked
 *    prefill cuts a long prompt into pieces; speculative decoding verifies
 *    several guessed tokens in one pass): several new query tokens per
 *    sequence, each attending causally to its context (varlen attention).
 *  - ipipp.com article on vLLM and PagedAttention (2026-09-14),
 *    section 二 "PagedAttention分页原理深度剖析": the KV cache is cut into
 *    fixed blocks of 16 tokens; a block table maps each logical block of a
 *    sequence to a physical block; the attention kernel walks the logical
 *    blocks, looks each one up in the table and reads that block's K/V.
 *    Paging only changes where K and V live, not the attention result.
 *  - bytelighting wiki entry "vLLM", 核心机制 / 工作原理, paragraph
 *    "Flattened 布局与 slot_mapping": slot_mapping sends each new token's
 *    logical position to a physical slot of the flattened block pool.
 *  - ai-maas.com "vLLM 深读：用 PagedAttention 撑起高并发 LLM 推理",
 *    section 先看浪费在哪里: blocks are logically contiguous but physically
 *    scattered, and sequences with a common prefix may point at the same
 *    physical blocks.
 *  - The same ai-maas.com page, section 引擎的分层结构 (quantisation list),
 *    names FP8; the e4m3 encoding itself follows the OCP 8-bit floating
 *    point specification (OFP8, E4M3: bias 7, no infinities, one NaN
 *    mantissa pattern, max 448).
 *
 * Conventions fixed where the pages are silent (each one is listed with its
 * reason in the repository's design notes):
 *  - Pool layout: separate K and V pools; slot s lives at block
 *    s / block_size, offset s % block_size.  Within a (block, KV head) tile
 *    the K pool stores each token row in 16-byte chunks of X = 16 / element
 *    size consecutive dimensions, chunk-major:
 *        K[block][kv_head][d / X][offset][d % X]
 *    and the V pool stores the tile dimension-major:
 *        V[block][kv_head][d][offset]
 *    (head_dim must be a multiple of X).
 *  - Query head h reads KV head h / (num_heads / num_kv_heads).
 *  - A slot_mapping entry of -1 means "skip this token".
 *  - context_lens[s] counts every cached token of sequence s, including the
 *    one written in the current step; a length of 0 yields an all-zero row.
 *
 * Parity pins: every function here is checked by tests against something
 * other than itself (library routines, closed forms, brute force, invariants,
 * and hand-worked fixtures).  No function is left "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Data type codes (the oracle's own numbering). */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2 };

/* Status codes (same meanings as the library's, numbered independently). */
enum {
    ORC_OK = 0,
    ORC_ERR_INVALID_ARG = 1,
    ORC_ERR_UNSUPPORTED = 2,
};

/* ------------------------------------------------------------------------ */
/* Scalar codecs                                                             */
/* ------------------------------------------------------------------------ */

static size_t elt_size(int dtype)
{
    switch (dtype) {
    case ORC_F32: return 4;
    case ORC_BF16: return 2;
    case ORC_FP8_E4M3: return 1;
    default: return 0;
    }
}

/* bfloat16 is the upper half of an IEEE binary32: widening is exact. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * OCP E4M3 decode.  Fields: sign (1 bit), exponent (4 bits, bias 7),
 * mantissa (3 bits).  Exponent field 0 is subnormal: m/8 * 2^(1-7).
 * Exponent 15 with mantissa 7 is NaN; there is no infinity.
 */
double oracle_fp8_e4m3_to_double(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - 7);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/*
 * OCP E4M3 encode of an already-scaled value y (saturating).
 * NaN keeps its sign as 0x7F / 0xFF.  |y| >= 448 (including infinity)
 * saturates to +-448.  Everything else goes to the nearest representable
 * value, ties to the even mantissa; the sign of zero is kept.
 * The arithmetic below is exact in double (y has 24 significant bits).
 */
uint8_t oracle_fp8_e4m3_encode(float y)
{
    uint8_t s = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (isnan(y))
        return (uint8_t)(s | 0x7F);
    if (a >= 448.0)
        return (uint8_t)(s | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: spacing 2^-9, codes 0..8 (8 is the smallest normal) */
        double m = nearbyint(a * 512.0); /* default rounding: to nearest, ties even */
        return (uint8_t)(s | (uint8_t)m);
    }
    {
        int fe;
        double fr = frexp(a, &fe); /* a = fr * 2^fe, fr in [0.5, 1) */
        int E = fe - 1;            /* a = (2 fr) * 2^E, 2 fr in [1, 2), E in [-6, 8] */
        double m = nearbyint((2.0 * fr - 1.0) * 8.0);
        if (m == 8.0) { /* rounded up into the next binade */
            m = 0.0;
            E += 1;
        }
        return (uint8_t)(s | ((E + 7) << 3) | (int)m);
    }
}

/* Quantise one input element: fp32 division by the scale, then encode. */
static uint8_t quantise(float x, float scale)
{
    float y = x / scale; /* IEEE binary32 division, correctly rounded */
    return oracle_fp8_e4m3_encode(y);
}

/* Read element i of a typed array as double (fp8 without its scale). */
static double load_as_double(const void* base, int dtype, size_t i)
{
    switch (dtype) {
    case ORC_F32: {
        float f;
        memcpy(&f, (const char*)base + 4 * i, 4);
        return (double)f;
    }
    case ORC_BF16: {
        uint16_t b;
        memcpy(&b, (const char*)base + 2 * i, 2);
        return oracle_bf16_to_double(b);
    }
    case ORC_FP8_E4M3:
        return oracle_fp8_e4m3_to_double(((const uint8_t*)base)[i]);
    default:
        return NAN;
    }
}

static float load_as_float(const void* base, int dtype, size_t i)
{
    /* exact for f32 and bf16 inputs (the only quantiser inputs) */
    return (float)load_as_double(base, dtype, i);
}

/* Vectorised helpers for the test suite. */
void oracle_fp8_e4m3_decode_n(const uint8_t* codes, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_fp8_e4m3_to_double(codes[i]);
}

void oracle_fp8_e4m3_quantise_n(const float* x, uint8_t* out, int64_t n, float scale)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = quantise(x[i], scale);
}

void oracle_bf16_to_double_n(const uint16_t* bits, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_double(bits[i]);
}

/* ------------------------------------------------------------------------ */
/* KV cache write through slot_mapping                                       */
/* ------------------------------------------------------------------------ */

/* Elements per 16-byte K chunk for a pool element type. */
static int k_chunk_elems(int dtype)
{
    size_t e = elt_size(dtype);
    return e ? (int)(16 / e) : 0;
}

/* Offset, in elements, of (block, head, offset-in-block, dim) in the K pool:
 * K[block][head][dim / X][offset][dim % X]. */
static size_t k_index(int64_t block, int head, int off, int d,
                      int num_kv_heads, int block_size, int head_dim, int X)
{
    size_t chunk = ((size_t)block * (size_t)num_kv_heads + (size_t)head) * (size_t)(head_dim / X)
                   + (size_t)(d / X);
    return (chunk * (size_t)block_size + (size_t)off) * (size_t)X + (size_t)(d % X);
}

/* Offset, in elements, of (block, head, offset-in-block, dim) in the V pool:
 * V[block][head][dim][offset]. */
static size_t v_index(int64_t block, int head, int off, int d,
                      int num_kv_heads, int block_size, int head_dim)
{
    return (((size_t)block * (size_t)num_kv_heads + (size_t)head) * (size_t)head_dim + (size_t)d)
           * (size_t)block_size + (size_t)off;
}

/*
 * Write num_tokens new tokens into the K and V pools.  Token i goes to slot
 * slot_mapping[i] (block = slot / block_size, offset = slot % block_size),
 * all heads and dims; -1 skips the token.  Same in/cache dtype: the bits are
 * copied.  fp8 cache with f32 or bf16 input: each element is quantised with
 * k_scale (K) or v_scale (V).
 * Errors: any slot below -1 or at/after num_blocks*block_size, a repeated
 * slot, a bad size, or an unsupported dtype pair.
 */
int oracle_kv_write(const void* k_new, const void* v_new, int in_dtype,
                    void* k_cache, void* v_cache, int cache_dtype,
                    const int32_t* slot_mapping, int32_t num_tokens,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, float k_scale, float v_scale)
{
    int quant;
    int64_t num_slots;
    uint8_t* seen;
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return ORC_ERR_INVALID_ARG;
    if (elt_size(in_dtype) == 0 || elt_size(cache_dtype) == 0)
        return ORC_ERR_UNSUPPORTED;
    if (in_dtype == cache_dtype)
        quant = 0;
    else if (cache_dtype == ORC_FP8_E4M3 && (in_dtype == ORC_F32 || in_dtype == ORC_BF16))
        quant = 1;
    else
        return ORC_ERR_UNSUPPORTED;
    if (quant && !(isfinite(k_scale) && k_scale > 0.0f && isfinite(v_scale) && v_scale > 0.0f))
        return ORC_ERR_INVALID_ARG;
    if (head_dim % k_chunk_elems(cache_dtype) != 0)
        return ORC_ERR_UNSUPPORTED;

    num_slots = (int64_t)num_blocks * block_size;
    seen = (uint8_t*)calloc((size_t)(num_slots > 0 ? num_slots : 1), 1);
    if (!seen)
        return ORC_ERR_INVALID_ARG;
    for (int32_t i = 0; i < num_tokens; ++i) {
        int32_t sl = slot_mapping[i];
        if (sl == -1)
            continue;
        if (sl < -1 || (int64_t)sl >= num_slots || seen[sl]) {
            free(seen);
            return ORC_ERR_INVALID_ARG;
        }
        seen[sl] = 1;
    }
    free(seen);

    for (int32_t i = 0; i < num_tokens; ++i) {
        int32_t sl = slot_mapping[i];
        int64_t block;
        int off;
        if (sl == -1)
            continue;
        block = sl / block_size;
        off = sl % block_size;
        for (int h = 0; h < num_kv_heads; ++h) {
            for (int d = 0; d < head_dim; ++d) {
                size_t src = ((size_t)i * num_kv_heads + h) * (size_t)head_dim + d;
                size_t kd = k_index(block, h, off, d, num_kv_heads, block_size, head_dim,
                                    k_chunk_elems(cache_dtype));
                size_t vd = v_index(block, h, off, d, num_kv_heads, block_size, head_dim);
                if (!quant) {
                    size_t es = elt_size(cache_dtype);
                    memcpy((char*)k_cache + kd * es, (const char*)k_new + src * es, es);
                    memcpy((char*)v_cache + vd * es, (const char*)v_new + src * es, es);
                } else {
                    ((uint8_t*)k_cache)[kd] = quantise(load_as_float(k_new, in_dtype, src), k_scale);
                    ((uint8_t*)v_cache)[vd] = quantise(load_as_float(v_new, in_dtype, src), v_scale);
                }
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Decode attention through the block table                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
    double* out;
    const void* q;
    int q_dtype;
    const void* k_cache;
    const void* v_cache;
    int cache_dtype;
    const int32_t* block_table;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    int32_t num_seqs, num_heads, num_kv_heads, head_dim, block_size;
    double scale, k_scale, v_scale;
    int32_t partition_size; /* 0: one pass over the whole context */
    int64_t next;           /* next (seq, head) work item */
    pthread_mutex_t lock;
} attn_job;

/* Dequantised K (is_v = 0) or V (is_v = 1) element of logical token t of
 * sequence s, KV head g, dimension d. */
static double kv_at(const attn_job* J, int is_v, int s, int g, int t, int d)
{
    int32_t block = J->block_table[(size_t)s * J->max_blocks_per_seq + t / J->block_size];
    int off = t % J->block_size;
    size_t idx = is_v ? v_index(block, g, off, d, J->num_kv_heads, J->block_size, J->head_dim)
                      : k_index(block, g, off, d, J->num_kv_heads, J->block_size, J->head_dim,
                                k_chunk_elems(J->cache_dtype));
    double x = load_as_double(is_v ? J->v_cache : J->k_cache, J->cache_dtype, idx);
    return J->cache_dtype == ORC_FP8_E4M3 ? x * (is_v ? J->v_scale : J->k_scale) : x;
}

/* Score of query row qr (its head h) against logical token t of sequence s:
 * scale * q[qr][h] . k_t.  In decode, query row qr is sequence s itself. */
static double score_row(const attn_job* J, int s, int64_t qr, int h, int g, int t)
{
    double acc = 0.0;
    size_t qbase = ((size_t)qr * J->num_heads + h) * (size_t)J->head_dim;
    for (int d = 0; d < J->head_dim; ++d)
        acc += load_as_double(J->q, J->q_dtype, qbase + d) * kv_at(J, 0, s, g, t, d);
    return J->scale * acc;
}

/* Score of query (s, h) against logical token t: scale * q . k_t */
static double score_at(const attn_job* J, int s, int h, int g, int t)
{
    double acc = 0.0;
    size_t qbase = ((size_t)s * J->num_heads + h) * (size_t)J->head_dim;
    for (int d = 0; d < J->head_dim; ++d)
        acc += load_as_double(J->q, J->q_dtype, qbase + d) * kv_at(J, 0, s, g, t, d);
    return J->scale * acc;
}

/*
 * Plain softmax attention of one query row over tokens [0, L):
 *   m = max_t score_t,  w_t = exp(score_t - m),  out = sum_t (w_t / sum w) v_t
 */
static void attend_one(const attn_job* J, int s, int h, double* row)
{
    int G = J->num_heads / J->num_kv_heads;
    int g = h / G;
    int L = J->context_lens[s];
    double* w;
    double m = -INFINITY, Z = 0.0;
    for (int d = 0; d < J->head_dim; ++d)
        row[d] = 0.0;
    if (L == 0)
        return;
    w = (double*)malloc(sizeof(double) * (size_t)L);
    for (int t = 0; t < L; ++t) {
        w[t] = score_at(J, s, h, g, t);
        if (w[t] > m)
            m = w[t];
    }
    for (int t = 0; t < L; ++t) {
        w[t] = exp(w[t] - m);
        Z += w[t];
    }
    for (int t = 0; t < L; ++t) {
        double p = w[t] / Z;
        for (int d = 0; d < J->head_dim; ++d)
            row[d] += p * kv_at(J, 1, s, g, t, d);
    }
    free(w);
}

/*
 * The same row computed split into partitions of P tokens, each reduced to
 * (m_p, l_p, acc_p) with acc_p = sum_t exp(score_t - m_p) v_t, then merged:
 *   M = max_p m_p,  out = sum_p exp(m_p - M) acc_p / sum_p exp(m_p - M) l_p.
 * Mathematically identical to attend_one; tests hold the two together.
 */
static void attend_one_split(const attn_job* J, int s, int h, double* row)
{
    int G = J->num_heads / J->num_kv_heads;
    int g = h / G;
    int L = J->context_lens[s];
    int P = J->partition_size;
    int np = (L + P - 1) / P;
    double *mp, *lp, *accp;
    double M = -INFINITY, den = 0.0;
    for (int d = 0; d < J->head_dim; ++d)
        row[d] = 0.0;
    if (L == 0)
        return;
    mp = (double*)malloc(sizeof(double) * (size_t)np);
    lp = (double*)calloc((size_t)np, sizeof(double));
    accp = (double*)calloc((size_t)np * (size_t)J->head_dim, sizeof(double));
    for (int p = 0; p < np; ++p) {
        int t0 = p * P, t1 = (p + 1) * P < L ? (p + 1) * P : L;
        mp[p] = -INFINITY;
        for (int t = t0; t < t1; ++t) {
            double sc = score_at(J, s, h, g, t);
            if (sc > mp[p])
                mp[p] = sc;
        }
        for (int t = t0; t < t1; ++t) {
            double w = exp(score_at(J, s, h, g, t) - mp[p]);
            lp[p] += w;
            for (int d = 0; d < J->head_dim; ++d)
                accp[(size_t)p * J->head_dim + d] += w * kv_at(J, 1, s, g, t, d);
        }
        if (mp[p] > M)
            M = mp[p];
    }
    for (int p = 0; p < np; ++p)
        den += exp(mp[p] - M) * lp[p];
    for (int p = 0; p < np; ++p) {
        double c = exp(mp[p] - M);
        for (int d = 0; d < J->head_dim; ++d)
            row[d] += c * accp[(size_t)p * J->head_dim + d] / den;
    }
    free(mp);
    free(lp);
    free(accp);
}

static void* attn_worker(void* arg)
{
    attn_job* J = (attn_job*)arg;
    int64_t total = (int64_t)J->num_seqs * J->num_heads;
    for (;;) {
        int64_t item;
        pthread_mutex_lock(&J->lock);
        item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= total)
            break;
        {
            int s = (int)(item / J->num_heads), h = (int)(item % J->num_heads);
            double* row = J->out + (size_t)item * J->head_dim;
            if (J->partition_size > 0)
                attend_one_split(J, s, h, row);
            else
                attend_one(J, s, h, row);
        }
    }
    return NULL;
}

/*
 * Several new query tokens per sequence (chunked prefill, speculative
 * verification).  Query row qr belongs to sequence s with cu[s] <= qr <
 * cu[s+1]; it is the i-th of the sequence's n = cu[s+1] - cu[s] new tokens,
 * which are the last n of its L cached tokens, so it sits at position
 * p = L - n + i and attends causally to tokens [0, p]:
 *   m = max_{t<=p} score_t,  out = sum_{t<=p} exp(score_t - m) v_t / sum_{t<=p} exp(score_t - m)
 */
static void attend_causal(const attn_job* J, int s, int64_t qr, int h, int limit, double* row)
{
    int G = J->num_heads / J->num_kv_heads;
    int g = h / G;
    double* w;
    double m = -INFINITY, Z = 0.0;
    for (int d = 0; d < J->head_dim; ++d)
        row[d] = 0.0;
    if (limit <= 0)
        return;
    w = (double*)malloc(sizeof(double) * (size_t)limit);
    for (int t = 0; t < limit; ++t) {
        w[t] = score_row(J, s, qr, h, g, t);
        if (w[t] > m)
            m = w[t];
    }
    for (int t = 0; t < limit; ++t) {
        w[t] = exp(w[t] - m);
        Z += w[t];
    }
    for (int t = 0; t < limit; ++t) {
        double pr = w[t] / Z;
        for (int d = 0; d < J->head_dim; ++d)
            row[d] += pr * kv_at(J, 1, s, g, t, d);
    }
    free(w);
}

int oracle_num_threads(int requested);

typedef struct {
    attn_job* J;
    const int32_t* cu;       /* [num_seqs + 1] */
    const int32_t* row_seq;  /* [num_rows] sequence of each query row */
    int64_t num_rows;
} varlen_job;

static void* varlen_worker(void* arg)
{
    varlen_job* V = (varlen_job*)arg;
    attn_job* J = V->J;
    int64_t total = V->num_rows * J->num_heads;
    for (;;) {
        int64_t item;
        pthread_mutex_lock(&J->lock);
        item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= total)
            break;
        {
            int64_t qr = item / J->num_heads;
            int h = (int)(item % J->num_heads);
            int s = V->row_seq[qr];
            int n = V->cu[s + 1] - V->cu[s];
            int i = (int)(qr - V->cu[s]);
            int pos = J->context_lens[s] - n + i;
            attend_causal(J, s, qr, h, pos + 1, J->out + (size_t)item * J->head_dim);
        }
    }
    return NULL;
}

/*
 * out[qr][h][:] (double) for every query row qr in [0, cu_seqlens_q[num_seqs])
 * as described at attend_causal.  Errors: as oracle_paged_attention, plus
 * cu_seqlens_q not starting at 0 or decreasing, or a sequence with more new
 * tokens than cached tokens.
 */
int oracle_paged_attention_varlen(double* out, const void* q, int q_dtype, const int32_t* cu_seqlens_q,
                                  const void* k_cache, const void* v_cache, int cache_dtype,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, float k_scale, float v_scale,
                                  int32_t num_threads)
{
    attn_job J;
    varlen_job V;
    int32_t* row_seq;
    int64_t rows;
    int nt;
    pthread_t* th;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0
        || num_blocks < 0 || max_blocks_per_seq < 0)
        return ORC_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0)
        return ORC_ERR_INVALID_ARG;
    if (!(q_dtype == ORC_F32 || q_dtype == ORC_BF16) || elt_size(cache_dtype) == 0)
        return ORC_ERR_UNSUPPORTED;
    if (head_dim % k_chunk_elems(cache_dtype) != 0)
        return ORC_ERR_UNSUPPORTED;
    if (cu_seqlens_q[0] != 0)
        return ORC_ERR_INVALID_ARG;
    for (int s = 0; s < num_seqs; ++s) {
        int64_t L = context_lens[s];
        int64_t n = (int64_t)cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        int64_t nb = (L + block_size - 1) / block_size;
        if (n < 0 || n > L || L > (int64_t)max_blocks_per_seq * block_size)
            return ORC_ERR_INVALID_ARG;
        for (int64_t j = 0; j < nb; ++j) {
            int32_t b = block_table[(size_t)s * max_blocks_per_seq + j];
            if (b < 0 || b >= num_blocks)
                return ORC_ERR_INVALID_ARG;
        }
    }
    rows = num_seqs > 0 ? cu_seqlens_q[num_seqs] : 0;
    row_seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows > 0 ? rows : 1));
    for (int s = 0; s < num_seqs; ++s)
        for (int32_t r = cu_seqlens_q[s]; r < cu_seqlens_q[s + 1]; ++r)
            row_seq[r] = s;

    J.out = out;
    J.q = q;
    J.q_dtype = q_dtype;
    J.k_cache = k_cache;
    J.v_cache = v_cache;
    J.cache_dtype = cache_dtype;
    J.block_table = block_table;
    J.max_blocks_per_seq = max_blocks_per_seq;
    J.context_lens = context_lens;
    J.num_seqs = num_seqs;
    J.num_heads = num_heads;
    J.num_kv_heads = num_kv_heads;
    J.head_dim = head_dim;
    J.block_size = block_size;
    J.scale = (double)scale;
    J.k_scale = (double)k_scale;
    J.v_scale = (double)v_scale;
    J.partition_size = 0;
    J.next = 0;
    pthread_mutex_init(&J.lock, NULL);
    V.J = &J;
    V.cu = cu_seqlens_q;
    V.row_seq = row_seq;
    V.num_rows = rows;

    nt = oracle_num_threads(num_threads);
    th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    for (int i = 0; i < nt; ++i)
        pthread_create(&th[i], NULL, varlen_worker, &V);
    for (int i = 0; i < nt; ++i)
        pthread_join(th[i], NULL);
    free(th);
    free(row_seq);
    pthread_mutex_destroy(&J.lock);
    return ORC_OK;
}

/* Number of worker threads actually used for a given request (0 = all cores). */
int oracle_num_threads(int requested)
{
    long n = requested > 0 ? requested : sysconf(_SC_NPROCESSORS_ONLN);
    if (n < 1)
        n = 1;
    if (n > 256)
        n = 256;
    return (int)n;
}

/*
 * out[s][h][:] (double) = softmax(scale * q[s][h] . K_s^T) V_s over the
 * context_lens[s] tokens found through block_table[s]; fp8 pools are
 * dequantised as code value * k_scale (K) or * v_scale (V).
 * partition_size > 0 selects the split-and-merge form (same result).
 * Errors: num_heads not a multiple of num_kv_heads, bad sizes, unsupported
 * dtypes, a length outside [0, max_blocks_per_seq * block_size], or a table
 * entry outside [0, num_blocks) among the first ceil(L / block_size) entries
 * of a row (later entries are padding and are never read).
 */
int oracle_paged_attention(double* out, const void* q, int q_dtype,
                           const void* k_cache, const void* v_cache, int cache_dtype,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, float scale, float k_scale, float v_scale,
                           int32_t partition_size, int32_t num_threads)
{
    attn_job J;
    int nt;
    pthread_t* th;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0
        || num_blocks < 0 || max_blocks_per_seq < 0 || partition_size < 0)
        return ORC_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0)
        return ORC_ERR_INVALID_ARG;
    if (!(q_dtype == ORC_F32 || q_dtype == ORC_BF16) || elt_size(cache_dtype) == 0)
        return ORC_ERR_UNSUPPORTED;
    if (head_dim % k_chunk_elems(cache_dtype) != 0)
        return ORC_ERR_UNSUPPORTED;
    for (int s = 0; s < num_seqs; ++s) {
        int64_t L = context_lens[s];
        int64_t nb = (L + block_size - 1) / block_size;
        if (L < 0 || L > (int64_t)max_blocks_per_seq * block_size)
            return ORC_ERR_INVALID_ARG;
        for (int64_t j = 0; j < nb; ++j) {
            int32_t b = block_table[(size_t)s * max_blocks_per_seq + j];
            if (b < 0 || b >= num_blocks)
                return ORC_ERR_INVALID_ARG;
        }
    }

    J.out = out;
    J.q = q;
    J.q_dtype = q_dtype;
    J.k_cache = k_cache;
    J.v_cache = v_cache;
    J.cache_dtype = cache_dtype;
    J.block_table = block_table;
    J.max_blocks_per_seq = max_blocks_per_seq;
    J.context_lens = context_lens;
    J.num_seqs = num_seqs;
    J.num_heads = num_heads;
    J.num_kv_heads = num_kv_heads;
    J.head_dim = head_dim;
    J.block_size = block_size;
    J.scale = (double)scale;
    J.k_scale = (double)k_scale;
    J.v_scale = (double)v_scale;
    J.partition_size = partition_size;
    J.next = 0;
    pthread_mutex_init(&J.lock, NULL);

    nt = oracle_num_threads(num_threads);
    th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    for (int i = 0; i < nt; ++i)
        pthread_create(&th[i], NULL, attn_worker, &J);
    for (int i = 0; i < nt; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return ORC_OK;
}
