/*
 * pa_decode.h - C ABI of libpa_decode.so: paged split-KV GQA/MQA decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (TensorRT-LLM XQA article, "TensorRT-LLM 源码完全拆解(二十九):
 * XQA 解码注意力内核", section 先把 decode 注意力的约束写清楚, its displayed
 * equation): one new query token per request; for request b, KV head h and each
 * of the G query heads g of that KV head,
 *
 *     out[b][h*G + g][:] = softmax(scale * q[b][h*G + g][:] . K_{b,h}^T) V_{b,h}
 *
 * where K_{b,h}, V_{b,h} are the first seq_lens[b] tokens of the request, stored
 * in fixed-size pages of a pool and found through a per-request block table
 * (same article, section "分页 KV: 页号怎么变成 TMA 坐标"; query heads of one KV
 * head are contiguous, section "GQA 的组内复用").  lse[b][hq] is the natural-log
 * log-sum-exp of the scaled logits (the FlashMLA walk-through returns (o, lse);
 * section 调度).  A request of length 0 gets out = 0 and lse = -inf.
 *
 * The sequence is split into chunks processed in parallel, each leaving a partial
 * (normalised output, lse) that a combine step merges (XQA article, section
 * "多块模式: 把一条序列沿 KV 切成几段"; FlashAttention tiling page, section 5
 * "Split-K 策略与 num_splits 启发式"; FlashMLA walk-through, sections 调度 and
 * 合并与性能账本).  Three calls, all enqueued on the caller's stream:
 *
 *   pa_decode_plan     split scheduler: writes the plan (which token ranges of which
 *                      request each workgroup processes) from device seq_lens
 *   pa_decode_run      split-KV decode kernel: writes final rows for requests done
 *                      in one chunk, partials (workspace) for the others
 *   pa_decode_combine  LSE-weighted merge of the partials into out / lse
 *
 * With PA_FLAG_FUSED_COMBINE (bf16 and fp8 page-head formats; MLA-656 with q_len 1 and
 * no sparse indices; the partial rows of one request, chunks x q_len x Hkv x G x Dv x 4
 * bytes with up to num_splits chunks, or 1024 under the balanced plan, below 2 GiB, else
 * PA_ERR_UNSUPPORTED) the merge runs inside pa_decode_run instead: the workgroup that
 * finishes the last chunk of a request merges that request's chunks (the XQA article's
 * "last CTA merges" variant, section "归约怎么记"), found with a device-scope counter per
 * (request, row group) kept in the plan buffer; then pa_decode_combine has nothing to do
 * and returns without launching.  The partials are written and read with
 * device-coherent (agent-scope) accesses, since the 8 XCD caches are not coherent with
 * each other; on MI355X the merging workgroup then waits for those stores, the counter
 * and the coherent reads in turn, which on small workloads costs more than the combine
 * launch it saves.
 * Ordering: the writers store their partials with the cache policy of relaxed agent-scope
 * atomics (sc1, 16 bytes per access), wait for their completion (s_waitcnt vmcnt(0)) and
 * then bump the counter with a relaxed agent-scope atomic; the merger reads with the same
 * policy.  This is not release/acquire in
 * the HIP memory model: it relies on gfx950 executing agent-scope atomics on memory that
 * is coherent across XCDs (the write-through policy those accesses carry), so a store
 * that has completed is visible to every later agent-scope load.  An agent-scope
 * release/acquire fence would write back / invalidate the whole L2 of the XCD instead
 * (measured 4x slower).  The library is built for gfx950 only, and the merge code refuses
 * to compile for any other target.
 *
 * Ownership: the caller allocates and owns every buffer (device memory for all
 * array arguments).  The library never allocates, frees or synchronises; it keeps
 * no state except a per-device compute-unit count.  Calls on one stream are
 * ordered by that stream; concurrent calls on different streams must not share a
 * plan, workspace or output buffer.
 *
 * Errors: arguments are validated on the host before anything is launched; a
 * non-PA_OK status means nothing was enqueued.  Device-side data (page ids,
 * seq_lens) is trusted, not checked: every page id a request can reach must be
 * < num_pages and seq_lens[b] <= max_pages_per_seq * page_size.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID = 1,      /* null pointer, non-positive size, misaligned pointer/stride */
    PA_ERR_UNSUPPORTED = 2,  /* a valid shape the library has no kernel for */
    PA_ERR_SIZE = 3,         /* plan or workspace smaller than the size query returned */
    PA_ERR_DEVICE = 4        /* a HIP call (device query, kernel launch) failed */
} pa_status;

typedef enum {
    /* bf16 K and V pools */
    PA_KV_BF16 = 0,
    /* OCP float8 e4m3 K and V pools; value = code * scale[page][kv_head], with separate
       fp32 scale tables for K and V (k_scale, v_scale: [num_pages][Hkv]) */
    PA_KV_FP8_E4M3_PAGE_HEAD = 1,
    /* MLA latent cache, 656 bytes per token (FlashMLA walk-through, section 数据加载):
       512 e4m3 codes | 4 fp32 scales (one per 128 codes) | 64 bf16 rope values.
       K = the 576 dequantised values, V = their first 512; v_pool must be NULL. */
    PA_KV_MLA656 = 2
} pa_kv_format;

enum {
    /* pa_decode_run merges the chunks itself; pa_decode_combine becomes a no-op.
       PA_KV_MLA656: with q_len 1 and topk 0 only (else PA_ERR_UNSUPPORTED). */
    PA_FLAG_FUSED_COMBINE = 1
};

typedef struct {
    int32_t B;                 /* requests (one query token each) */
    int32_t Hkv;               /* KV heads; query heads Hq = Hkv * G */
    int32_t G;                 /* query heads per KV head (GQA group size; Hkv = 1: MQA);
                                  bf16 / fp8: 1..16; MLA: a multiple of 16 up to 128 */
    int32_t D;                 /* q / K head dim: 64 or 128 (bf16, fp8), 576 (MLA) */
    int32_t Dv;                /* V / out head dim: = D, or 512 for MLA */
    int32_t page_size;         /* tokens per page: 16, 32, 64, 128 or 256 */
    int32_t num_pages;         /* pages in the pool */
    int32_t max_pages_per_seq; /* columns of block_table */
    /* pool strides in storage units (bf16: 2-byte elements; fp8 and MLA: bytes).
       Token t of request b, KV head h starts at
       pool + page * s_page + h * s_head + (t % page_size) * s_tok
       with page = block_table[b][t / page_size].  HND [page][Hkv][P][D]:
       s_page = Hkv*P*D, s_head = P*D, s_tok = D.  NHD [page][P][Hkv][D]:
       s_page = P*Hkv*D, s_head = D, s_tok = Hkv*D.  MLA: s_tok = 656 (656 .. 2^20
       accepted, else PA_ERR_INVALID / PA_ERR_UNSUPPORTED), s_head unused.
       Every stride times the unit size must be a multiple of 16 bytes. */
    int64_t s_page, s_head, s_tok;
    int32_t q_len;             /* query tokens per request (a linear draft, token i sees keys
                                  [0, L - q_len + i]): 1..64, G * q_len <= 256 for bf16/fp8,
                                  <= 1024 for MLA */
    int32_t num_splits;        /* 0: balanced split scheduling; s > 0: s chunks per request */
    int32_t kv_format;         /* pa_kv_format */
    int32_t flags;             /* 0 or PA_FLAG_FUSED_COMBINE; other bits: PA_ERR_INVALID */
    int32_t window;            /* sliding window W > 0: the query token at position p sees
                                  keys [max(0, p - W + 1), p]; tiles before the window are
                                  never read (XQA article, section "分页 KV: 页号怎么变成
                                  TMA 坐标").  0: off */
    int32_t topk;              /* sparse decode (PA_KV_MLA656, q_len 1, no window): each
                                  request attends to the topk key positions listed in
                                  `indices` (FlashMLA walk-through, section 调度).  0: off */
} pa_decode_desc;

/*
 * Split scheduler.  With plan == NULL: size query only - writes the plan and
 * workspace sizes in bytes (either pointer may be NULL), touches no device memory.
 * Otherwise enqueues the plan kernel on `stream` (a hipStream_t; NULL = default
 * stream), which reads seq_lens[B] (int32, device) and writes the plan.
 * *plan_bytes must then hold the plan buffer's size (PA_ERR_SIZE if smaller).
 *
 * num_splits = s > 0: request b is cut into s chunks of ceil(ceil(L_b/64)/s)
 * 64-token tiles each (FlashAttention tiling page, section 5.3; trailing chunks may
 * be empty).  num_splits = 0: the tiles of all requests are laid end to end and cut
 * into equal contiguous parts, one workgroup per (part, KV head), a few per compute
 * unit (FlashMLA walk-through, section 调度); a request is cut where a part ends.
 *
 * The plan stays valid while the desc and seq_lens are unchanged, so one plan can
 * serve every layer of a decode step.  The plan's last words are the fused-combine
 * counters (B x row groups, a row group being the G query heads of one KV head, or 64
 * query heads for PA_KV_MLA656); the plan kernel zeroes them.
 */
pa_status pa_decode_plan(const pa_decode_desc *desc, const int32_t *seq_lens, void *plan,
                         size_t *plan_bytes, size_t *workspace_bytes, void *stream);

/*
 * Split-KV decode.  Enqueues the decode kernel.
 *   q           [B][Hq][D] bf16
 *   k_pool      K pool (or the MLA656 pool), layout given by the desc strides
 *   v_pool      V pool; NULL for PA_KV_MLA656
 *   k_scale, v_scale  [num_pages][Hkv] fp32 for PA_KV_FP8_E4M3_PAGE_HEAD, else NULL
 *   block_table [B][max_pages_per_seq] int32; seq_lens [B] int32 (must be the values
 *               the plan was built from)
 *   indices     desc->topk > 0: [B][topk] int32 key positions per request; entries
 *               outside [0, seq_lens[b]) are skipped, a position listed twice counts
 *               twice.  Else NULL.
 *   sinks       [Hkv * G] fp32 attention-sink logits (units of scale * q . k) or NULL.
 *               A sink joins the softmax denominator once and carries no value (XQA
 *               article, section "一个容易漏掉的细节: attention sink"): out = sum_t
 *               e^{s_t} v_t / (e^{sink} + sum_t e^{s_t}), lse = ln(e^{sink} + sum_t e^{s_t}).
 *               Pass the same pointer to pa_decode_combine.
 *   scale       logit scale; <= 0 selects 1/sqrt(D)
 *   out         [B][Hq][Dv] bf16; lse [B][Hq] fp32 (natural log)
 *   plan        written by pa_decode_plan for the same desc (flags may differ).  With
 *               PA_FLAG_FUSED_COMBINE the kernel counts finished chunks in the plan's
 *               counter words and leaves them at zero when it completes, so runs that
 *               share one plan must be ordered (one stream), never concurrent.
 *   workspace   >= the size pa_decode_plan reported (fp32 partials), 16-byte aligned
 * Without PA_FLAG_FUSED_COMBINE, rows of requests that the plan cuts into several
 * chunks (and rows of length-0 requests under the balanced rule) are only complete
 * after pa_decode_combine; with it, every row is complete when the kernel ends.
 */
pa_status pa_decode_run(const pa_decode_desc *desc, void *plan, const void *q,
                        const void *k_pool, const void *v_pool, const float *k_scale,
                        const float *v_scale, const int32_t *block_table,
                        const int32_t *seq_lens, const int32_t *indices, const float *sinks,
                        float scale, void *out, float *lse, void *workspace, void *stream);

/*
 * Combine.  For every request cut into several chunks (and every request of length
 * 0) merges the chunk partials: M = max_i lse_i, lse = M + ln sum_i exp(lse_i - M),
 * out = sum_i exp(lse_i - lse) * O_i (XQA article, section "归约怎么记", merge
 * equation, written for normalised partials).  Requests done in one chunk are left
 * as pa_decode_run wrote them.  sinks: the pointer given to pa_decode_run (its sink
 * joins each merged row once).  A no-op launch-free call when num_splits == 1 or the
 * desc has PA_FLAG_FUSED_COMBINE.
 */
pa_status pa_decode_combine(const pa_decode_desc *desc, const void *plan, const void *workspace,
                            const float *sinks, void *out, float *lse, void *stream);

/*
 * KV append: writes n_new new tokens per request into their pages, the step before
 * attention (XQA article, section "一次 decode step 的完整时序": attention reads a
 * cache that already holds the step's K/V).  seq_lens[b] (device) is the length AFTER
 * the append; new token j of request b goes to position seq_lens[b] - n_new + j, whose
 * page block_table[b][pos / page_size] the caller has already assigned.
 *   k_new, v_new  [B][n_new][Hkv][D] bf16, 16-byte aligned (PA_KV_MLA656: k_new
 *                 [B][n_new][576] bf16, v_new and v_pool NULL)
 *   k_pool, v_pool  written in place; k_scale, v_scale [num_pages][Hkv] fp32, read and
 *                 written (PA_KV_FP8_E4M3_PAGE_HEAD), else NULL
 * PA_KV_BF16: plain copy.  PA_KV_FP8_E4M3_PAGE_HEAD: each (page, KV head) scale is the
 * running max|x| / 448 of the values the page has received.  A page whose first slot
 * receives a new token starts fresh (scale = amax / 448 of its new values, 1 if all are
 * 0); otherwise scale = max(old, amax / 448), and when it grows the page's older codes
 * are re-encoded with it (e4m3(fp32(fp32(decode(c) * old) / scale)), one more rounding
 * each).  Codes are OCP E4M3FN, round to nearest even, saturating at +-448.
 * PA_KV_MLA656: per token, one scale per 128-value tile = max|x| / 448 (1 if 0), codes
 * e4m3(fp32(x / scale)), the 64 rope values copied as bf16.
 * Pages that receive new tokens must belong to a single request; requests with
 * seq_lens[b] < n_new are skipped.  n_new <= 65535.
 */
pa_status pa_kv_append(const pa_decode_desc *desc, int32_t n_new, const void *k_new,
                       const void *v_new, const int32_t *block_table, const int32_t *seq_lens,
                       void *k_pool, void *v_pool, float *k_scale, float *v_scale, void *stream);

/*
 * No-allocation decode step, for callers that cannot allocate device memory (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid hipMalloc):
 * pa_decode_plan + pa_decode_run + pa_decode_combine in one call, with the plan and the
 * chunk partials in a buffer the library holds in device memory instead of caller
 * buffers: PA_NOALLOC_SCRATCH_BYTES per device, reserved when the library is loaded on
 * that device and kept until the process ends.  Arguments as for pa_decode_run (flags,
 * q_len, window, topk and sinks included); the result is bit-identical to the three-call
 * sequence.  Every call on one device shares that buffer and leaves its contents there:
 * calls that overlap on one device (other streams, other threads) race on it, so the
 * caller must order them.  The plan is rebuilt on every call (the plan kernel also
 * clears the fused-combine counters it holds).  PA_ERR_SIZE: this desc's plan (rounded
 * up to 256 bytes) and partials need more than PA_NOALLOC_SCRATCH_BYTES; nothing is
 * enqueued.  No allocation, free or synchronisation.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_noalloc(const pa_decode_desc *desc, const void *q, const void *k_pool,
                            const void *v_pool, const float *k_scale, const float *v_scale,
                            const int32_t *block_table, const int32_t *seq_lens,
                            const int32_t *indices, const float *sinks, float scale, void *out,
                            float *lse, void *stream);

/* Number of workgroups along the part axis that pa_decode_run launches for `desc`
   on the current device (B * num_splits, or the balanced part count). */
pa_status pa_decode_num_parts(const pa_decode_desc *desc, int32_t *num_parts);

/* Static string for a status code (a pa_status value; any other int gives "unknown status").
   The parameter is an int, not the enum type, so that any value a caller passes is valid. */
const char *pa_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* PA_DECODE_H */
