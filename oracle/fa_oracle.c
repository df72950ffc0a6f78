/*
 * CPU oracle for causal grouped-query attention (f16 / bf16 / q4_0 K and V).
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load this library. It shares no code, header, table or helper with the HIP path, and
 * the HIP path never calls it.
 *
 * What it computes is the plain definition that the pages check their kernels against:
 *   O = softmax(scale * Q K^T + causal mask) V
 * evaluated as an f32 product, a softmax and a second product (mlxcel PR #2306, commit
 * message 2 and "Test plan", whose causal checks use such an f32 reference; mi210-llm-stack
 * "Build FlashAttention (CK backend) on gfx90a", Verification: the fused kernel compared with
 * torch's scaled_dot_product_attention). Every query row is computed on its own: the row's
 * visible scores, their maximum, exp of the shifted scores, their sum, and the weighted sum of
 * V rows. No tiling, no online softmax, no deferred frame.
 *
 * Conventions (readings of the pages, each listed in the design notes):
 *   - layouts are [B, S, H, D] contiguous; query head h reads K/V head h / (Hq / Hkv)
 *     (consecutive grouping of "GQA 32/8", mlxcel PR commit message 1);
 *   - query i sits at absolute position i + offset and, when causal, sees key j iff
 *     j <= i + offset (the mlxcel PR #2306 measures query chunks of 2048 tokens against key
 *     ranges of 2K to 16K, which this reads as the chunk being the last Sq positions, so
 *     offset = Sk - Sq there);
 *   - a row that sees no key outputs zeros;
 *   - q4_0 ("-ctk q4_0 -ctv q4_0", mi210-llm-stack page 1): 18-byte blocks of 32 head-dim
 *     elements, a little-endian f16 scale d then 16 bytes where byte t holds the 4-bit code of
 *     element t (low nibble) and of element t+16 (high nibble); element value (c - 8) * d.
 *
 * All inputs are first converted exactly to f32: f16 and bf16 widen exactly, and (c - 8) * d is
 * exact in f32 because a 4-bit integer times an 11-bit significand needs at most 15 bits.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_Q4_0 = 2 };

enum {
    ORC_OK = 0,
    ORC_ERR_ARG = -1,
    ORC_ERR_NOMEM = -2,
};

/* ---------------------------------------------------------------------------------------- */
/* scalar conversions, written from the IEEE 754 binary16 and bfloat16 definitions           */
/* ---------------------------------------------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static float half_bits_to_float(uint16_t h)
{
    const int sign = h >> 15;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    float mag;
    if (e == 0)
        mag = ldexpf((float)f, -24);               /* subnormal: f * 2^-24 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexpf((float)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of a binary32. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return x;
}

/* Round a float to the nearest binary16, ties to even. */
static uint16_t float_to_half_bits_rne(float x)
{
    const uint16_t s = signbit(x) ? 0x8000u : 0u;
    const float a = fabsf(x);
    if (isnan(x))
        return (uint16_t)(s | 0x7E00u);
    if (isinf(a))
        return (uint16_t)(s | 0x7C00u);
    if (a == 0.0f)
        return s;
    int k;
    frexpf(a, &k);
    k -= 1;                                         /* a lies in [2^k, 2^(k+1)) */
    if (k < -14) {
        /* below the smallest normal the spacing is 2^-24; a count of 1024 is the smallest
           normal, whose bit pattern is also 1024 */
        const float n = nearbyintf(ldexpf(a, 24));
        return (uint16_t)(s | (uint16_t)n);
    }
    /* spacing 2^(k-10): the significand count n lies in [1024, 2048]; n == 2048 carries into
       the exponent field, which the sum below does by itself */
    const float n = nearbyintf(ldexpf(a, 10 - k));
    const uint32_t bits = ((uint32_t)(k + 15) << 10) + ((uint32_t)n - 1024u);
    if (bits >= 0x7C00u)
        return (uint16_t)(s | 0x7C00u);
    return (uint16_t)(s | bits);
}

/* One q4_0 block: 18 bytes -> 32 floats, value (c - 8) * d. */
static void q4_0_block_to_float(const uint8_t *blk, float *out)
{
    const float d = half_bits_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
    for (int t = 0; t < 16; ++t) {
        const int lo = blk[2 + t] & 15;
        const int hi = blk[2 + t] >> 4;
        out[t] = (float)(lo - 8) * d;
        out[t + 16] = (float)(hi - 8) * d;
    }
}

int orc_dequant_q4_0(const uint8_t *blocks, int64_t n_blocks, float *out_f32, uint16_t *out_f16)
{
    if (!blocks || n_blocks < 0 || (!out_f32 && !out_f16))
        return ORC_ERR_ARG;
    for (int64_t b = 0; b < n_blocks; ++b) {
        float x[32];
        q4_0_block_to_float(blocks + 18 * b, x);
        for (int t = 0; t < 32; ++t) {
            if (out_f32)
                out_f32[32 * b + t] = x[t];
            if (out_f16)
                out_f16[32 * b + t] = float_to_half_bits_rne(x[t]);
        }
    }
    return ORC_OK;
}

int orc_half_to_float(const uint16_t *h, int64_t n, float *out)
{
    if (!h || !out || n < 0)
        return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i)
        out[i] = half_bits_to_float(h[i]);
    return ORC_OK;
}

int orc_float_to_half(const float *x, int64_t n, uint16_t *out)
{
    if (!x || !out || n < 0)
        return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i)
        out[i] = float_to_half_bits_rne(x[i]);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------------- */
/* q4_0 cache writer                                                                          */
/* ---------------------------------------------------------------------------------------- */
/* The pages name the q4_0 cache type (mi210-llm-stack page 1, "-ctk q4_0 -ctv q4_0") without
 * defining it; the benchmark configurations give the scale d = max|x| / 8 and the element value
 * (c - 8) * d. The rest is a reading: d is that quotient rounded to the nearest binary16, ties
 * to even; an element's code is c = clamp(round_half_away(x / d) + 8, 0, 15) with x / d the
 * correctly rounded f32 quotient (so the element +max|x| gives 16, clamped to 15); every code is
 * 8 when d == 0. Source elements (f32, f16 or bf16) are widened exactly to f32 first; non-finite
 * inputs and max|x| / 8 above the largest binary16 are outside the reading. */
enum { ORC_SRC_F32 = 0, ORC_SRC_F16 = 1, ORC_SRC_BF16 = 2 };

static void q4_0_quantize_block(const float *x, uint8_t *blk)
{
    float amax = 0.0f;
    for (int t = 0; t < 32; ++t)
        if (fabsf(x[t]) > amax)
            amax = fabsf(x[t]);
    const uint16_t dbits = float_to_half_bits_rne(amax / 8.0f);
    const float d = half_bits_to_float(dbits);
    int c[32];
    for (int t = 0; t < 32; ++t) {
        int v = 8;
        if (d != 0.0f) {
            v = (int)roundf(x[t] / d) + 8;
            v = v < 0 ? 0 : (v > 15 ? 15 : v);
        }
        c[t] = v;
    }
    blk[0] = (uint8_t)(dbits & 0xFFu);
    blk[1] = (uint8_t)(dbits >> 8);
    for (int t = 0; t < 16; ++t)
        blk[2 + t] = (uint8_t)(c[t] | (c[t + 16] << 4));
}

/* n_blocks blocks of 32 consecutive source elements -> n_blocks q4_0 blocks of 18 bytes. */
int orc_quantize_q4_0(const void *x, int x_dtype, int64_t n_blocks, uint8_t *blocks)
{
    if (n_blocks < 0 || (n_blocks > 0 && (!x || !blocks)) ||
        (x_dtype != ORC_SRC_F32 && x_dtype != ORC_SRC_F16 && x_dtype != ORC_SRC_BF16))
        return ORC_ERR_ARG;
    for (int64_t b = 0; b < n_blocks; ++b) {
        float v[32];
        for (int t = 0; t < 32; ++t) {
            const int64_t e = 32 * b + t;
            if (x_dtype == ORC_SRC_F32)
                v[t] = ((const float *)x)[e];
            else if (x_dtype == ORC_SRC_F16)
                v[t] = half_bits_to_float(((const uint16_t *)x)[e]);
            else
                v[t] = bf16_bits_to_float(((const uint16_t *)x)[e]);
        }
        q4_0_quantize_block(v, blocks + 18 * b);
    }
    return ORC_OK;
}

/* Widen `rows` rows of D elements stored as `dtype` into a new f32 buffer. Every element is
 * widened on its own, so splitting the loop over threads changes no value. */
static float *upcast_rows(const void *src, int dtype, int64_t rows, int D)
{
    float *dst = (float *)malloc(sizeof(float) * (size_t)rows * (size_t)D);
    if (!dst)
        return NULL;
    const int64_t n = rows * D;
    if (dtype == ORC_F16) {
        const uint16_t *s = (const uint16_t *)src;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            dst[i] = half_bits_to_float(s[i]);
    } else if (dtype == ORC_BF16) {
        const uint16_t *s = (const uint16_t *)src;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            dst[i] = bf16_bits_to_float(s[i]);
    } else {
        const uint8_t *s = (const uint8_t *)src;
        const int nb = D / 32;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            for (int b = 0; b < nb; ++b)
                q4_0_block_to_float(s + (r * nb + b) * 18, dst + r * D + 32 * b);
    }
    return dst;
}

typedef struct {
    const float *Q, *K, *V;
    int B, Hq, Hkv, Sq, Sk, D, causal;
    int64_t offset;
    float scale;
} problem;

/* Number of keys row i can see: keys 0 .. n-1. */
static int64_t visible_keys(const problem *p, int64_t i)
{
    if (!p->causal)
        return p->Sk;
    int64_t n = i + p->offset + 1;
    if (n < 0)
        n = 0;
    if (n > p->Sk)
        n = p->Sk;
    return n;
}

/* Softmax probabilities of flattened row r = (b * Sq + i) * Hq + h into p[0 .. n-1];
   returns n, the number of visible keys. */
static int64_t row_probs(const problem *p, int64_t r, float *prob)
{
    const int64_t h = r % p->Hq;
    const int64_t i = (r / p->Hq) % p->Sq;
    const int64_t b = r / ((int64_t)p->Hq * p->Sq);
    const int64_t g = h / (p->Hq / p->Hkv);
    const float *q = p->Q + r * p->D;
    const int64_t n = visible_keys(p, i);
    if (n == 0)
        return 0;
    /* scores: s_j = scale * sum_d q_d k_jd */
    for (int64_t j = 0; j < n; ++j) {
        const float *k = p->K + ((b * p->Sk + j) * p->Hkv + g) * p->D;
        float acc = 0.0f;
        for (int d = 0; d < p->D; ++d)
            acc += q[d] * k[d];
        prob[j] = p->scale * acc;
    }
    /* softmax over the visible keys */
    float m = prob[0];
    for (int64_t j = 1; j < n; ++j)
        if (prob[j] > m)
            m = prob[j];
    float l = 0.0f;
    for (int64_t j = 0; j < n; ++j) {
        prob[j] = expf(prob[j] - m);
        l += prob[j];
    }
    for (int64_t j = 0; j < n; ++j)
        prob[j] = prob[j] / l;
    return n;
}

/* Output row r: o_d = sum_j p_j v_jd (zeros when the row sees no key). */
static void row_output(const problem *p, int64_t r, float *prob, float *o)
{
    const int64_t h = r % p->Hq;
    const int64_t b = r / ((int64_t)p->Hq * p->Sq);
    const int64_t g = h / (p->Hq / p->Hkv);
    const int64_t n = row_probs(p, r, prob);
    for (int d = 0; d < p->D; ++d)
        o[d] = 0.0f;
    for (int64_t j = 0; j < n; ++j) {
        const float *v = p->V + ((b * p->Sk + j) * p->Hkv + g) * p->D;
        for (int d = 0; d < p->D; ++d)
            o[d] += prob[j] * v[d];
    }
}

static int check_cache_dtype(int dtype, int D)
{
    if (dtype != ORC_F16 && dtype != ORC_BF16 && dtype != ORC_Q4_0)
        return ORC_ERR_ARG;
    if (dtype == ORC_Q4_0 && D % 32)
        return ORC_ERR_ARG;
    return ORC_OK;
}

static int check_args(const void *q, const void *k, const void *v, int q_dtype, int k_dtype,
                      int v_dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D)
{
    if (!q || !k || !v)
        return ORC_ERR_ARG;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Sk < 0 || D <= 0 || Hq % Hkv)
        return ORC_ERR_ARG;
    if (q_dtype != ORC_F16 && q_dtype != ORC_BF16)
        return ORC_ERR_ARG;
    if (check_cache_dtype(k_dtype, D) || check_cache_dtype(v_dtype, D))
        return ORC_ERR_ARG;
    return ORC_OK;
}

/*
 * Attention for a list of query rows. Q is [B, Sq, Hq, D] stored as q_dtype; K and V are
 * [B, Sk, Hkv, D] stored as k_dtype and v_dtype (q4_0: [B, Sk, Hkv, D/32] blocks of 18
 * bytes). The two cache types are independent settings (mi210-llm-stack, "FlashAttention
 * on gfx90a", sets them with one flag per cache, -ctk and -ctv): each tensor is widened to
 * f32 by its own type, and nothing after that depends on either type.
 * rows[] holds flattened row indices (b * Sq + i) * Hq + h; with rows == NULL every row is
 * computed in order and `out` takes the [B, Sq, Hq, D] layout. out is f32 [n_rows, D].
 * threads <= 0 lets OpenMP choose.
 */
int orc_attention_kv(const void *q, const void *k, const void *v, int q_dtype, int k_dtype,
                     int v_dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                     int64_t offset, float scale, const int64_t *rows, int64_t n_rows,
                     float *out, int threads)
{
    int rc = check_args(q, k, v, q_dtype, k_dtype, v_dtype, B, Hq, Hkv, Sq, Sk, D);
    if (rc)
        return rc;
    if (!out)
        return ORC_ERR_ARG;
    const int64_t total = (int64_t)B * Sq * Hq;
    if (!rows)
        n_rows = total;
    for (int64_t t = 0; rows && t < n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= total)
            return ORC_ERR_ARG;

    problem p = {0};
    p.Q = upcast_rows(q, q_dtype, total, D);
    p.K = upcast_rows(k, k_dtype, (int64_t)B * Sk * Hkv, D);
    p.V = upcast_rows(v, v_dtype, (int64_t)B * Sk * Hkv, D);
    rc = (p.Q && p.K && p.V) ? ORC_OK : ORC_ERR_NOMEM;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Sk = Sk; p.D = D;
    p.causal = causal; p.offset = offset; p.scale = scale;

    if (rc == ORC_OK) {
#ifdef _OPENMP
        if (threads <= 0)
            threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
#endif
        {
            float *prob = (float *)malloc(sizeof(float) * (size_t)(Sk > 0 ? Sk : 1));
            if (!prob) {
                rc = ORC_ERR_NOMEM;
            } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
                for (int64_t t = 0; t < n_rows; ++t)
                    row_output(&p, rows ? rows[t] : t, prob, out + t * D);
                free(prob);
            }
        }
    }
    free((void *)p.Q);
    free((void *)p.K);
    free((void *)p.V);
    return rc;
}

/* orc_attention_kv with one type for both caches. */
int orc_attention(const void *q, const void *k, const void *v, int q_dtype, int kv_dtype,
                  int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int64_t offset,
                  float scale, const int64_t *rows, int64_t n_rows, float *out, int threads)
{
    return orc_attention_kv(q, k, v, q_dtype, kv_dtype, kv_dtype, B, Hq, Hkv, Sq, Sk, D, causal,
                            offset, scale, rows, n_rows, out, threads);
}

/* Softmax probabilities of one query row over all Sk keys (zeros for keys it cannot see). */
int orc_probs(const void *q, const void *k, int q_dtype, int kv_dtype,
              int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int64_t offset,
              float scale, int64_t row, float *p_out)
{
    int rc = check_args(q, k, k, q_dtype, kv_dtype, kv_dtype, B, Hq, Hkv, Sq, Sk, D);
    if (rc)
        return rc;
    const int64_t total = (int64_t)B * Sq * Hq;
    if (!p_out || row < 0 || row >= total)
        return ORC_ERR_ARG;
    problem p = {0};
    p.Q = upcast_rows(q, q_dtype, total, D);
    p.K = upcast_rows(k, kv_dtype, (int64_t)B * Sk * Hkv, D);
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Sk = Sk; p.D = D;
    p.causal = causal; p.offset = offset; p.scale = scale;
    if (!p.Q || !p.K) {
        rc = ORC_ERR_NOMEM;
    } else {
        for (int64_t j = 0; j < Sk; ++j)
            p_out[j] = 0.0f;
        row_probs(&p, row, p_out);
    }
    free((void *)p.Q);
    free((void *)p.K);
    return rc;
}
