/*
 * Decode-attention oracle (test infrastructure only; see oracle.c).
 * Nothing in the product library includes this header.
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_KV_BF16 = 0, ORACLE_KV_FP8_PAGE_HEAD = 1, ORACLE_KV_MLA656 = 2 };

typedef struct {
    int32_t B, Hkv, G, D, Dv;
    int32_t page_size, num_pages, max_pages;
    /* pool strides, in storage units: bf16 elements (2 B) for ORACLE_KV_BF16,
       bytes for ORACLE_KV_FP8_PAGE_HEAD and ORACLE_KV_MLA656 */
    int64_t s_page, s_head, s_tok;
    int32_t kv_format;
    int32_t q_len;   /* query tokens per request (1: plain decode) */
    int32_t window;  /* sliding window in tokens (0: off) */
    int32_t topk;    /* sparse: key positions per request listed in `indices` (0: dense) */
} oracle_desc;

double oracle_bf16_to_f64(uint16_t bits);
double oracle_e4m3_to_f64(uint8_t code);
void oracle_mla656_unpack(const uint8_t *tok, double *k576);

int oracle_threads(int nthreads);

int oracle_decode(const oracle_desc *d, const uint16_t *q, const void *k_pool,
                  const void *v_pool, const float *k_scale, const float *v_scale,
                  const int32_t *block_table, const int32_t *seq_lens, const int32_t *indices,
                  const float *sinks, double scale, const uint8_t *pair_mask, double *out,
                  double *lse, int nthreads);

int oracle_ranges(const oracle_desc *d, const uint16_t *q, const void *k_pool,
                  const void *v_pool, const float *k_scale, const float *v_scale,
                  const int32_t *block_table, const int32_t *seq_lens, const int32_t *indices,
                  double scale, int n, const int32_t *rb,
                  const int32_t *rt0, const int32_t *rt1, double *m, double *l, double *Ot,
                  int nthreads);

void oracle_merge(int n, int rows, int Dv, const double *m, const double *l, const double *Ot,
                  double *O, double *lse);

uint8_t oracle_e4m3_encode(float x);
void oracle_e4m3_encode_n(const float *x, uint8_t *codes, int64_t n);
int oracle_kv_append(const oracle_desc *d, int n_new, const uint16_t *k_new,
                     const uint16_t *v_new, const int32_t *block_table, const int32_t *seq_lens,
                     void *k_pool, void *v_pool, float *k_scale, float *v_scale);

void oracle_e4m3_decode_n(const uint8_t *codes, double *out, int64_t n);
void oracle_bf16_decode_n(const uint16_t *bits, double *out, int64_t n);
void oracle_mla656_unpack_n(const uint8_t *toks, double *k576, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
