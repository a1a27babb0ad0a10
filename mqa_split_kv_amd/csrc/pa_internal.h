// Internal declarations shared by the host API and the kernel translation units of
// libpa_decode.so.  Each kernel file defines its kernels and the host launcher that
// starts them; nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pa_decode.h"

namespace pa {

// Scheduling granule: a request's tokens are cut into chunks at multiples of this.
constexpr int kTileTokens = 64;
constexpr int kPlanMagic = 0x50414450;
constexpr int kPlanHeaderWords = 8;
constexpr int kMaxBatch = 4096;       // plan kernel keeps per-request prefix sums in LDS
constexpr int kMaxPlanParts = 1024;   // and the balanced rule's per-part prefix

// Plan buffer (int32 words):
//   [0] magic  [1] mode (0 fixed splits, 1 balanced)  [2] B  [3] num_parts
//   [4] num_items  [5] tile tokens  [6] max_items  [7] 0
//   part_begin[num_parts + 1] | chunk_off[B + 1] | items[max_items][4] = {b, tok0, tok1, flags}
//   | counters[B][n_rowgroups]
//   flags bit 0: the item is its request's only chunk and writes the final row.
//   counters: chunks of (request, row group) finished so far in a fused-combine run;
//   zeroed by the plan kernel, returned to zero by the run that uses them.  A row group
//   is the G query rows of one KV head (bf16 / fp8) or one 64-head group (MLA).
struct PlanLayout {
    int mode;
    int B;
    int num_parts;
    int max_items;
    int part_begin_off;
    int chunk_off_off;
    int items_off;
    int counters_off;
    int n_counters;
    size_t words;
};

inline PlanLayout plan_layout(int B, int n_rowgroups, int num_splits, int num_parts)
{
    PlanLayout L;
    L.mode = num_splits > 0 ? 0 : 1;
    L.B = B;
    L.num_parts = num_parts;
    L.max_items = num_splits > 0 ? B * num_splits : num_parts + B;
    L.part_begin_off = kPlanHeaderWords;
    L.chunk_off_off = L.part_begin_off + num_parts + 1;
    L.items_off = L.chunk_off_off + B + 1;
    L.counters_off = L.items_off + 4 * L.max_items;
    L.n_counters = B * n_rowgroups;
    L.words = (size_t)L.counters_off + (size_t)L.n_counters;
    return L;
}

// Workspace: normalised fp32 partial outputs [max_items][q_len][Hkv][G][Dv], then
// (256-byte aligned) fp32 partial lse [max_items][q_len][Hkv][G] in natural log.  The
// partial row of query row qr = qi * Hq + hq in chunk c is c * q_len * Hq + qr.
inline size_t ws_o_bytes(int max_items, int qrows, int Dv)
{
    size_t b = (size_t)max_items * qrows * Dv * 4;
    return (b + 255) & ~(size_t)255;
}
inline size_t ws_bytes(int max_items, int qrows, int Dv)
{
    return ws_o_bytes(max_items, qrows, Dv) + (size_t)max_items * qrows * 4;
}

struct DecodeArgs {
    const uint16_t *q;          // [B][q_len][Hq][D] bf16
    const uint8_t *k_pool;      // byte pointers; strides below are in bytes
    const uint8_t *v_pool;
    const float *k_scale;       // [num_pages][Hkv] (fp8 formats)
    const float *v_scale;
    const int32_t *block_table; // [B][max_pages]
    const int32_t *plan;
    uint16_t *out;              // [B][q_len][Hq][Dv] bf16
    float *lse;                 // [B][q_len][Hq]
    float *ws_o;
    float *ws_lse;
    int64_t s_page_b, s_head_b, s_tok_b;   // pool strides in bytes
    const int32_t *seq_lens;    // [B]
    const int32_t *indices;     // [B][topk] key positions (sparse) or null
    const float *sinks;         // [Hq] sink logits (natural units) or null
    int B, Hkv, G, D, Dv, max_pages, page_shift;
    int q_len;                  // query tokens per request; query token i sees keys
                                // [0, L - q_len + i + 1)
    int window;                 // sliding window (0: off)
    int topk;                   // sparse key slots per request (0: dense)
    int num_parts, part_begin_off, items_off, chunk_off_off;
    int fixed_splits;           // s > 0: a fixed-split plan, part p is exactly item p (and
                                // request b's chunks are b*s .. b*s+s-1); 0: balanced
    int32_t *counters;          // plan counter words; non-null: fused combine
    float scale_log2;           // logit scale * log2(e)
    int kv_format;
};

hipError_t launch_plan(const int32_t *seq_lens, int32_t *plan, const PlanLayout &L,
                       const pa_decode_desc *d, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_mla(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_append(const pa_decode_desc *d, int n_new, const void *k_new, const void *v_new,
                         const int32_t *block_table, const int32_t *seq_lens, void *k_pool,
                         void *v_pool, float *k_scale, float *v_scale, hipStream_t stream);
hipError_t launch_combine(const int32_t *plan, const float *ws_o, const float *ws_lse,
                          const float *sinks, uint16_t *out, float *lse, int B, int Hkv, int G,
                          int q_len, int Dv, int chunk_off_off, int fixed_splits, int kv_format,
                          hipStream_t stream);

}  // namespace pa
