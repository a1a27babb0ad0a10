/*
 * Decode-attention oracle: the plain CPU definition of paged GQA/MQA decode
 * attention, in fp64.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product path never does.  It shares
 * no code, header, table or constant with the HIP library.
 *
 * What it computes (source: "TensorRT-LLM 源码完全拆解(二十九): XQA 解码注意力内核",
 * section 先把 decode 注意力的约束写清楚, the displayed equation):
 *
 *   out[b, h*G + g, :] = softmax( scale * q[b, h*G+g, :] . K_{b,h}^T ) V_{b,h}
 *
 * for every request b, KV head h and grouped query head g < G.  The query heads
 * of one KV head are contiguous (same page, section "GQA 的组内复用", the output
 * offset headGrpSize * idxHeadGrp + g).  K_{b,h} and V_{b,h} are the first
 * seq_lens[b] tokens of the request, gathered page by page: token t lives in
 * physical page block_table[b][t / P] at slot t % P (same page, section
 * "分页 KV: 页号怎么变成 TMA 坐标").
 *
 * lse is the natural log of sum_t exp(scale * q . k_t) (the FlashMLA walk-through
 * returns (o, lse) for merging; the pages do not define it further, so the plain
 * log-sum-exp of the scaled logits is used).  An empty token range gives out = 0
 * and lse = -inf.
 *
 * Several query tokens per request (speculative decoding with a linear draft; XQA
 * article, section "投机解码: XQA 的第二个工作负载"): the q_len draft tokens are the
 * last q_len positions of the request, their K/V already in the cache (the KV append
 * happens before attention, same article, section "一次 decode step 的完整时序"), and
 * a chain draft lets draft token i see the cached context and the draft tokens up to
 * itself: query token i (0-based) attends to tokens [0, L - q_len + i + 1).  q is
 * [B][q_len][Hq][D], out [B][q_len][Hq][Dv], lse [B][q_len][Hq].
 *
 * Variants on the same definition (readings of the pages, which name these without
 * formulas):
 *  - sliding window W > 0 (XQA article, section "分页 KV: 页号怎么变成 TMA 坐标": the
 *    window only looks at the last W tokens, so leading pages are skipped): the query
 *    token at position p attends to [max(0, p - W + 1), p + 1).
 *  - attention sink (XQA article, section "一个容易漏掉的细节: attention sink"): a
 *    per-query-head logit sink[hq], in the units of scale * q . k, that joins the
 *    softmax denominator once and carries no value: out = sum_t e^{s_t} v_t /
 *    (e^{sink} + sum_t e^{s_t}) and lse = ln(e^{sink} + sum_t e^{s_t}).  It is the
 *    merge of one more partial (m = sink, l = 1, O = 0), the form used below.
 *  - sparse top-k (FlashMLA walk-through, section 调度: the decode call takes sparse
 *    indices): one query token per request, which attends to the key positions
 *    indices[b][0 .. topk) of its request; entries outside [0, L) are skipped and a
 *    position listed twice counts twice.
 *
 * Pins: see tests/test_oracle.py (dense library attention, closed forms,
 * invariances, the rescale worked example, all 256 e4m3 codes).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "oracle.h"

/* ------------------------------------------------------------------------ */
/* Element decoders                                                          */
/* ------------------------------------------------------------------------ */

/* bfloat16 -> fp64: the 16 stored bits are the top half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary32 stored as 4 little-endian bytes -> fp64. */
static double f32_bytes_to_f64(const uint8_t *p)
{
    float f;
    memcpy(&f, p, sizeof f);
    return (double)f;
}

/*
 * OCP FP8 E4M3 ("e4m3fn", the float8_e4m3 of the pages) -> fp64.
 * 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no infinities; the
 * all-ones exponent+mantissa pattern (0x7F / 0xFF) is NaN; largest finite
 * magnitude 448 (the XQA page's kE4M3_MAX, section "Hopper 路径上 V 不做显式反量化").
 *   exponent field 0 : (-1)^s * 2^-6 * (m / 8)          (subnormal)
 *   otherwise        : (-1)^s * 2^(e-7) * (1 + m / 8)
 */
double oracle_e4m3_to_f64(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/*
 * MLA 656-byte token (FlashMLA walk-through, section 数据加载, byte-layout table):
 *   bytes [0, 512)   : 512 e4m3 codes, the first 512 of the 576 latent dims
 *   bytes [512, 528) : 4 fp32 scales, one per 128 consecutive codes
 *   bytes [528, 656) : 64 bf16 values, the last 64 dims (rope part, not quantized)
 * The key is the 576-vector nope || rope; the value is the first 512 dims
 * (the value shares the dequantized latent with the key).
 */
void oracle_mla656_unpack(const uint8_t *tok, double *k576)
{
    for (int j = 0; j < 512; j++)
        k576[j] = oracle_e4m3_to_f64(tok[j]) * f32_bytes_to_f64(tok + 512 + 4 * (j / 128));
    for (int r = 0; r < 64; r++) {
        uint16_t bits = (uint16_t)(tok[528 + 2 * r] | ((uint16_t)tok[528 + 2 * r + 1] << 8));
        k576[512 + r] = oracle_bf16_to_f64(bits);
    }
}

/* ------------------------------------------------------------------------ */
/* Token fetch through the block table                                      */
/* ------------------------------------------------------------------------ */

/* Physical page and in-page slot of logical token t of request b. */
static void locate(const oracle_desc *d, const int32_t *block_table, int b, int t,
                   int64_t *page, int64_t *slot)
{
    *page = block_table[(int64_t)b * d->max_pages + t / d->page_size];
    *slot = t % d->page_size;
}

/*
 * Dequantised key (is_v = 0) or value (is_v = 1) vector of token t, KV head h,
 * request b, written to x[0 .. D) or x[0 .. Dv).
 *   bf16 : exact widening
 *   fp8  : e4m3 code times the fp32 scale of that (page, KV head); K and V have
 *          their own scale tables
 *   MLA  : see oracle_mla656_unpack; V = first Dv dims of K
 */
static void fetch(const oracle_desc *d, const void *k_pool, const void *v_pool,
                  const float *k_scale, const float *v_scale, const int32_t *block_table,
                  int b, int h, int t, int is_v, double *x)
{
    int64_t page, slot;
    locate(d, block_table, b, t, &page, &slot);
    int64_t off = page * d->s_page + (int64_t)h * d->s_head + slot * d->s_tok;
    int n = is_v ? d->Dv : d->D;
    if (d->kv_format == ORACLE_KV_BF16) {
        const uint16_t *p = (const uint16_t *)(is_v ? v_pool : k_pool) + off;
        for (int i = 0; i < n; i++)
            x[i] = oracle_bf16_to_f64(p[i]);
    } else if (d->kv_format == ORACLE_KV_FP8_PAGE_HEAD) {
        const uint8_t *p = (const uint8_t *)(is_v ? v_pool : k_pool) + off;
        double s = (double)(is_v ? v_scale : k_scale)[page * d->Hkv + h];
        for (int i = 0; i < n; i++)
            x[i] = oracle_e4m3_to_f64(p[i]) * s;
    } else {
        double k576[576];
        oracle_mla656_unpack((const uint8_t *)k_pool + off, k576);
        for (int i = 0; i < n; i++)
            x[i] = k576[i];
    }
}

/* ------------------------------------------------------------------------ */
/* One (range, KV head): the partial state of the XQA multi-block page       */
/* ------------------------------------------------------------------------ */

/*
 * For request b, KV head h and token range [t0, t1), compute for each grouped
 * head g the partial triple of the XQA page (section "归约怎么记: 每个子序列一个
 * 「和-最大值」对"):
 *   m_g   = max_t s_t                          (local max)
 *   l_g   = sum_t exp(s_t - m_g)               (local denominator)
 *   Ot_g  = sum_t exp(s_t - m_g) * v_t         (local unnormalised output)
 * with s_t = scale * q_g . k_t.  An empty range gives m = -inf, l = 0, Ot = 0.
 * Two passes over the tokens: logits and their max first, then the weights.
 */
static int range_state(const oracle_desc *d, const uint16_t *q, const void *k_pool,
                       const void *v_pool, const float *k_scale, const float *v_scale,
                       const int32_t *block_table, double scale, int b, int h, int qi, int t0,
                       int t1, int tlo, const int32_t *idx, int L, double *m, double *l,
                       double *Ot)
{
    const int G = d->G, D = d->D, Dv = d->Dv;
    if (!idx && t0 < tlo)
        t0 = tlo;
    const int n = t1 > t0 ? t1 - t0 : 0;
    for (int g = 0; g < G; g++) {
        m[g] = -INFINITY;
        l[g] = 0.0;
        for (int i = 0; i < Dv; i++)
            Ot[(int64_t)g * Dv + i] = 0.0;
    }
    if (n == 0)
        return 0;

    double *qf = (double *)malloc(sizeof(double) * (size_t)G * D);
    double *s = (double *)malloc(sizeof(double) * (size_t)G * n);
    double *x = (double *)malloc(sizeof(double) * (size_t)(D > Dv ? D : Dv));
    if (!qf || !s || !x) {
        free(qf);
        free(s);
        free(x);
        return -1;
    }
    const int Hq = d->Hkv * G;
    for (int g = 0; g < G; g++)
        for (int i = 0; i < D; i++)
            qf[(int64_t)g * D + i] = oracle_bf16_to_f64(
                q[(((int64_t)b * d->q_len + qi) * Hq + (int64_t)h * G + g) * D + i]);

    /* token of range slot u: position t0 + u, or the listed position idx[t0 + u] (sparse;
       -1 when it lies outside the request) */
#define RANGE_TOKEN(u) (idx ? ((idx[t0 + (u)] >= 0 && idx[t0 + (u)] < L) ? idx[t0 + (u)] : -1) : t0 + (u))
    /* pass 1: logits */
    for (int u = 0; u < n; u++) {
        const int t = RANGE_TOKEN(u);
        if (t < 0)
            continue;
        fetch(d, k_pool, v_pool, k_scale, v_scale, block_table, b, h, t, 0, x);
        for (int g = 0; g < G; g++) {
            double acc = 0.0;
            for (int i = 0; i < D; i++)
                acc += qf[(int64_t)g * D + i] * x[i];
            double st = scale * acc;
            s[(int64_t)g * n + u] = st;
            if (st > m[g])
                m[g] = st;
        }
    }
    /* pass 2: weights, denominator, weighted values */
    for (int u = 0; u < n; u++) {
        const int t = RANGE_TOKEN(u);
        if (t < 0)
            continue;
        fetch(d, k_pool, v_pool, k_scale, v_scale, block_table, b, h, t, 1, x);
        for (int g = 0; g < G; g++) {
            double w = exp(s[(int64_t)g * n + u] - m[g]);
            l[g] += w;
            for (int i = 0; i < Dv; i++)
                Ot[(int64_t)g * Dv + i] += w * x[i];
        }
    }
#undef RANGE_TOKEN
    free(qf);
    free(s);
    free(x);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Public entry points                                                       */
/* ------------------------------------------------------------------------ */

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int oracle_threads(int nthreads) { return set_threads(nthreads); }

/* Causal limit of query token qi of a request of length L: it sees tokens [0, lim). */
static int causal_limit(const oracle_desc *d, int L, int qi)
{
    const int lim = L - (d->q_len - 1 - qi);
    return lim > 0 ? lim : 0;
}

/* First token query token qi sees under the sliding window (0 without one). */
static int window_start(const oracle_desc *d, int L, int qi)
{
    if (d->window <= 0)
        return 0;
    const int lo = L - d->q_len + qi - d->window + 1;
    return lo > 0 ? lo : 0;
}

/*
 * Whole-request attention for every (b, h) with pair_mask[b*Hkv+h] != 0
 * (pair_mask NULL: all pairs):  out = Ot / l,  lse = m + ln l, for each query token.
 * out is [B][q_len][Hq][Dv], lse is [B][q_len][Hq]; rows of skipped pairs are left
 * untouched.
 */
int oracle_decode(const oracle_desc *d, const uint16_t *q, const void *k_pool,
                  const void *v_pool, const float *k_scale, const float *v_scale,
                  const int32_t *block_table, const int32_t *seq_lens, const int32_t *indices,
                  const float *sinks, double scale, const uint8_t *pair_mask, double *out,
                  double *lse, int nthreads)
{
    const int B = d->B, Hkv = d->Hkv, G = d->G, Dv = d->Dv, Hq = Hkv * G, nq = d->q_len;
    if (d->topk > 0 && (nq != 1 || !indices))
        return -1;
    int err = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t pr = 0; pr < (int64_t)B * Hkv * nq; pr++) {
        const int b = (int)(pr / ((int64_t)Hkv * nq));
        const int h = (int)((pr / nq) % Hkv), qi = (int)(pr % nq);
        if (pair_mask && !pair_mask[(int64_t)b * Hkv + h])
            continue;
        double *m = (double *)malloc(sizeof(double) * (size_t)G);
        double *l = (double *)malloc(sizeof(double) * (size_t)G);
        double *Ot = (double *)malloc(sizeof(double) * (size_t)G * Dv);
        const int L = seq_lens[b];
        int rc = -1;
        if (m && l && Ot) {
            if (d->topk > 0)
                rc = range_state(d, q, k_pool, v_pool, k_scale, v_scale, block_table, scale, b, h,
                                 qi, 0, d->topk, 0, indices + (int64_t)b * d->topk, L, m, l, Ot);
            else
                rc = range_state(d, q, k_pool, v_pool, k_scale, v_scale, block_table, scale, b, h,
                                 qi, 0, causal_limit(d, L, qi), window_start(d, L, qi), NULL, L,
                                 m, l, Ot);
        }
        if (rc != 0) {
            err |= 1;
        } else {
            for (int g = 0; g < G; g++) {
                const int64_t row = ((int64_t)b * nq + qi) * Hq + (int64_t)h * G + g;
                if (sinks) {
                    /* merge with the sink's partial (m = sink, l = 1, O = 0) */
                    const double ms[2] = {m[g], (double)sinks[h * G + g]};
                    const double ls[2] = {l[g], 1.0};
                    double *ot2 = (double *)calloc(2 * (size_t)Dv, sizeof(double));
                    if (!ot2) {
                        err |= 1;
                        continue;
                    }
                    memcpy(ot2, Ot + (int64_t)g * Dv, sizeof(double) * (size_t)Dv);
                    oracle_merge(2, 1, Dv, ms, ls, ot2, out + row * Dv, lse + row);
                    free(ot2);
                } else if (l[g] > 0.0) {
                    for (int i = 0; i < Dv; i++)
                        out[row * Dv + i] = Ot[(int64_t)g * Dv + i] / l[g];
                    lse[row] = m[g] + log(l[g]);
                } else {
                    for (int i = 0; i < Dv; i++)
                        out[row * Dv + i] = 0.0;
                    lse[row] = -INFINITY;
                }
            }
        }
        free(m);
        free(l);
        free(Ot);
    }
    return err ? -1 : 0;
}

/*
 * Partial triples for a list of n token ranges (request rb[i], tokens
 * [rt0[i], rt1[i])), for every query token and KV head; query token qi only sees the
 * part of the range below its causal limit (seq_lens may be NULL when q_len == 1):
 *   m, l : [n][q_len][Hkv][G]     Ot : [n][q_len][Hkv][G][Dv]
 */
int oracle_ranges(const oracle_desc *d, const uint16_t *q, const void *k_pool,
                  const void *v_pool, const float *k_scale, const float *v_scale,
                  const int32_t *block_table, const int32_t *seq_lens, const int32_t *indices,
                  double scale, int n, const int32_t *rb, const int32_t *rt0, const int32_t *rt1,
                  double *m, double *l, double *Ot, int nthreads)
{
    const int Hkv = d->Hkv, G = d->G, Dv = d->Dv, nq = d->q_len;
    if ((nq > 1 || d->window > 0 || d->topk > 0) && !seq_lens)
        return -1;
    if (d->topk > 0 && !indices)
        return -1;
    int err = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t pr = 0; pr < (int64_t)n * nq * Hkv; pr++) {
        const int i = (int)(pr / ((int64_t)nq * Hkv));
        const int qi = (int)((pr / Hkv) % nq), h = (int)(pr % Hkv);
        int t1 = rt1[i], tlo = 0;
        const int L = seq_lens ? seq_lens[rb[i]] : 0;
        const int32_t *idx = d->topk > 0 ? indices + (int64_t)rb[i] * d->topk : NULL;
        if (!idx && seq_lens) {
            const int lim = causal_limit(d, L, qi);
            if (t1 > lim)
                t1 = lim;
            tlo = window_start(d, L, qi);
        }
        if (range_state(d, q, k_pool, v_pool, k_scale, v_scale, block_table, scale, rb[i], h, qi,
                        rt0[i], t1, tlo, idx, L, m + pr * G, l + pr * G,
                        Ot + pr * (int64_t)G * Dv) != 0)
            err |= 1;
    }
    return err ? -1 : 0;
}

/*
 * Merge of n partial triples into one result, for `rows` independent rows of
 * width Dv (XQA page, section "归约怎么记", the merge equation):
 *   m   = max_i m_i
 *   l   = sum_i l_i * exp(m_i - m)
 *   O   = (1 / l) * sum_i Ot_i * exp(m_i - m)
 * and lse = m + ln l.  Partials with m_i = -inf (empty ranges) carry no weight;
 * if every partial is empty, O = 0 and lse = -inf (the rule of never forming
 * -inf - (-inf), pipelining page, section 三, "分数可以早算").
 *   m, l : [n][rows]   Ot : [n][rows][Dv]   O : [rows][Dv]   lse : [rows]
 */
void oracle_merge(int n, int rows, int Dv, const double *m, const double *l, const double *Ot,
                  double *O, double *lse)
{
    for (int r = 0; r < rows; r++) {
        double mm = -INFINITY;
        for (int i = 0; i < n; i++)
            if (m[(int64_t)i * rows + r] > mm)
                mm = m[(int64_t)i * rows + r];
        double *o = O + (int64_t)r * Dv;
        for (int k = 0; k < Dv; k++)
            o[k] = 0.0;
        if (mm == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double ll = 0.0;
        for (int i = 0; i < n; i++) {
            double mi = m[(int64_t)i * rows + r];
            if (mi == -INFINITY)
                continue;
            double w = exp(mi - mm);
            ll += l[(int64_t)i * rows + r] * w;
            const double *oti = Ot + ((int64_t)i * rows + r) * Dv;
            for (int k = 0; k < Dv; k++)
                o[k] += oti[k] * w;
        }
        for (int k = 0; k < Dv; k++)
            o[k] /= ll;
        lse[r] = mm + log(ll);
    }
}

/* Vector helpers for the Python wrapper and the codec pins. */
void oracle_e4m3_decode_n(const uint8_t *codes, double *outv, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        outv[i] = oracle_e4m3_to_f64(codes[i]);
}

void oracle_bf16_decode_n(const uint16_t *bits, double *outv, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        outv[i] = oracle_bf16_to_f64(bits[i]);
}

void oracle_mla656_unpack_n(const uint8_t *toks, double *k576, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        oracle_mla656_unpack(toks + i * 656, k576 + i * 576);
}

/* ------------------------------------------------------------------------ */
/* KV append (the step before attention)                                    */
/* ------------------------------------------------------------------------ */
/*
 * The new tokens' K/V are written into their pages before attention reads them
 * (XQA article, section "一次 decode step 的完整时序": the cache already holds the
 * step's tokens; the append itself happens upstream).  The pages fix no append
 * procedure for quantised pages, so the following reading is taken:
 *
 *  - n_new new tokens per request; seq_lens are the lengths after the append, new
 *    token j of request b goes to position seq_lens[b] - n_new + j.
 *  - bf16 pools: plain copy.
 *  - fp8 page-head pools: one scale per (page, KV head), kept equal to the running
 *    max|x| / 448 of the values the page has received.  For each page that gets new
 *    tokens (slots [s0, s1) of it), in position order, with fp32 arithmetic:
 *        amax  = max |x| over the new values of that page and head
 *        s0 = 0 (fresh page): scale = amax > 0 ? amax / 448 : 1
 *        s0 > 0:              scale = max(old scale, amax / 448); when it grows, each
 *                             older code c of the page is re-encoded as
 *                             e4m3(fp32(fp32(decode(c) * old) / scale))
 *        new codes            e4m3(fp32(x / scale))
 *    K and V have their own scales.
 *  - MLA 656-byte tokens (FlashMLA walk-through, section 数据加载): per token and
 *    128-value tile, scale = amax > 0 ? amax / 448 : 1, codes e4m3(fp32(x / scale)),
 *    the 64 rope values copied as bf16.
 *  - e4m3(.) is the OCP E4M3FN encoding with round-to-nearest-even, saturating at
 *    +-448 (the largest finite value; the format has no infinity).
 */

/* OCP E4M3FN encoding of an fp32 value: round to nearest, ties to even; magnitudes
   >= 448 give +-448; NaN gives 0x7F.  The representable magnitudes are k * 2^-9 for
   k < 8 (subnormals) and (8 + m) * 2^(E-3) for m < 8 in the binade [2^E, 2^(E+1)). */
uint8_t oracle_e4m3_encode(float xf)
{
    if (isnan(xf))
        return 0x7F;
    const uint8_t s = signbit(xf) ? 0x80 : 0x00;
    const double a = fabs((double)xf);
    if (a >= 448.0)
        return s | 0x7E;
    int E;
    if (a < ldexp(1.0, -6)) {
        E = -6;                      /* subnormal spacing 2^-9 */
    } else {
        frexp(a, &E);                /* a = f 2^E', f in [0.5, 1): binade 2^(E'-1) */
        E -= 1;
    }
    const double qstep = ldexp(1.0, E - 3);
    const double r = rint(a / qstep) * qstep;    /* a / qstep is exact; rint: ties to even */
    if (r == 0.0)
        return s;
    if (r < ldexp(1.0, -6))
        return s | (uint8_t)(r / ldexp(1.0, -9));
    int e;
    const double f = frexp(r, &e);               /* r = (2f) 2^(e-1), 2f in [1, 2) */
    const int ebits = (e - 1) + 7;
    const int m = (int)((2.0 * f - 1.0) * 8.0);
    return s | (uint8_t)(ebits << 3) | (uint8_t)m;
}

static float bf16_to_f32(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp8 page-head append of one pool (K or V) for request b, KV head h. */
static void append_fp8_pool(const oracle_desc *d, int n_new, const uint16_t *x_new,
                            const int32_t *block_table, int b, int h, int L, uint8_t *pool,
                            float *scales)
{
    const int P = d->page_size, D = d->D, Hkv = d->Hkv;
    const int first = L - n_new;
    int j = 0;
    while (j < n_new) {
        const int pos0 = first + j;
        const int lp = pos0 / P, s0 = pos0 % P;
        int s1 = s0;
        while (j + (s1 - s0) < n_new && s1 < P)
            s1++;
        const int64_t page = block_table[(int64_t)b * d->max_pages + lp];
        float amax = 0.0f;
        for (int t = 0; t < s1 - s0; t++)
            for (int i = 0; i < D; i++) {
                const float v = fabsf(bf16_to_f32(x_new[(((int64_t)b * n_new + j + t) * Hkv + h) * D + i]));
                if (v > amax)
                    amax = v;
            }
        float *sc = &scales[page * Hkv + h];
        const float cand = amax > 0.0f ? amax / 448.0f : 1.0f;
        float scale;
        if (s0 == 0) {
            scale = cand;
        } else {
            const float old = *sc;
            const float grown = amax / 448.0f;
            scale = grown > old ? grown : old;
            if (scale > old) {
                for (int t = 0; t < s0; t++) {
                    uint8_t *row = pool + page * d->s_page + (int64_t)h * d->s_head + (int64_t)t * d->s_tok;
                    for (int i = 0; i < D; i++) {
                        const float xo = (float)oracle_e4m3_to_f64(row[i]) * old;
                        row[i] = oracle_e4m3_encode(xo / scale);
                    }
                }
            }
        }
        for (int t = 0; t < s1 - s0; t++) {
            uint8_t *row = pool + page * d->s_page + (int64_t)h * d->s_head + (int64_t)(s0 + t) * d->s_tok;
            for (int i = 0; i < D; i++) {
                const float x = bf16_to_f32(x_new[(((int64_t)b * n_new + j + t) * Hkv + h) * D + i]);
                row[i] = oracle_e4m3_encode(x / scale);
            }
        }
        *sc = scale;
        j += s1 - s0;
    }
}

/*
 * Append n_new tokens per request.  k_new, v_new: [B][n_new][Hkv][D] bf16 (MLA:
 * k_new [B][n_new][576] bf16, v_new unused).  Pools and scale tables are updated in
 * place.  Returns -1 if a request is shorter than n_new.
 */
int oracle_kv_append(const oracle_desc *d, int n_new, const uint16_t *k_new,
                     const uint16_t *v_new, const int32_t *block_table, const int32_t *seq_lens,
                     void *k_pool, void *v_pool, float *k_scale, float *v_scale)
{
    const int B = d->B, Hkv = d->Hkv, D = d->D, P = d->page_size;
    for (int b = 0; b < B; b++)
        if (seq_lens[b] < n_new)
            return -1;
    for (int b = 0; b < B; b++) {
        const int L = seq_lens[b];
        if (d->kv_format == ORACLE_KV_MLA656) {
            for (int j = 0; j < n_new; j++) {
                const int pos = L - n_new + j;
                const int64_t page = block_table[(int64_t)b * d->max_pages + pos / P];
                uint8_t *tok = (uint8_t *)k_pool + page * d->s_page + (int64_t)(pos % P) * d->s_tok;
                const uint16_t *x = k_new + ((int64_t)b * n_new + j) * 576;
                for (int tile = 0; tile < 4; tile++) {
                    float amax = 0.0f;
                    for (int i = 0; i < 128; i++) {
                        const float v = fabsf(bf16_to_f32(x[128 * tile + i]));
                        if (v > amax)
                            amax = v;
                    }
                    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
                    for (int i = 0; i < 128; i++)
                        tok[128 * tile + i] = oracle_e4m3_encode(bf16_to_f32(x[128 * tile + i]) / scale);
                    memcpy(tok + 512 + 4 * tile, &scale, 4);
                }
                for (int r = 0; r < 64; r++) {
                    tok[528 + 2 * r] = (uint8_t)(x[512 + r] & 0xFF);
                    tok[528 + 2 * r + 1] = (uint8_t)(x[512 + r] >> 8);
                }
            }
            continue;
        }
        for (int h = 0; h < Hkv; h++) {
            if (d->kv_format == ORACLE_KV_BF16) {
                for (int j = 0; j < n_new; j++) {
                    const int pos = L - n_new + j;
                    const int64_t page = block_table[(int64_t)b * d->max_pages + pos / P];
                    const int64_t off = page * d->s_page + (int64_t)h * d->s_head + (int64_t)(pos % P) * d->s_tok;
                    memcpy((uint16_t *)k_pool + off, k_new + (((int64_t)b * n_new + j) * Hkv + h) * D, 2 * (size_t)D);
                    memcpy((uint16_t *)v_pool + off, v_new + (((int64_t)b * n_new + j) * Hkv + h) * D, 2 * (size_t)D);
                }
            } else {
                append_fp8_pool(d, n_new, k_new, block_table, b, h, L, (uint8_t *)k_pool, k_scale);
                append_fp8_pool(d, n_new, v_new, block_table, b, h, L, (uint8_t *)v_pool, v_scale);
            }
        }
    }
    return 0;
}

void oracle_e4m3_encode_n(const float *x, uint8_t *codes, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        codes[i] = oracle_e4m3_encode(x[i]);
}
