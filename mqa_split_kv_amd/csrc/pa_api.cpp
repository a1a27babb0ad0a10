// Host side of libpa_decode.so: argument validation, size queries and kernel launches
// for the three C entry points declared in include/pa_decode.h.
#include <math.h>
#include <string.h>

#include <atomic>

#include "pa_internal.h"

namespace {

using pa::PlanLayout;

// Decode workgroups per compute unit for the balanced plan (one 4-wave workgroup per
// unit keeps enough KV loads in flight to stream at the HBM read ceiling).
#ifndef PA_WGS_PER_CU
#define PA_WGS_PER_CU 1
#endif

constexpr int kMaxDevices = 64;
constexpr int kMaxQLen = 64;
constexpr int kMaxAppendTokens = 65535;     // grid y of the MLA append
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (queried once per device).
int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < kMaxDevices) {
        int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
        return -1;
    if (dev < kMaxDevices) g_cu_count[dev].store(v, std::memory_order_relaxed);
    return v;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

int elem_bytes(int fmt) { return fmt == PA_KV_BF16 ? 2 : 1; }

// Shape checks shared by all entry points (no pointers).
pa_status check_desc(const pa_decode_desc *d)
{
    if (!d) return PA_ERR_INVALID;
    if (d->B <= 0 || d->Hkv <= 0 || d->G <= 0 || d->D <= 0 || d->Dv <= 0) return PA_ERR_INVALID;
    if (d->page_size <= 0 || d->num_pages <= 0 || d->max_pages_per_seq <= 0) return PA_ERR_INVALID;
    if (d->s_page < 0 || d->s_head < 0 || d->s_tok <= 0) return PA_ERR_INVALID;
    if (d->num_splits < 0 || (d->flags & ~(int32_t)PA_FLAG_FUSED_COMBINE) != 0 || d->q_len <= 0)
        return PA_ERR_INVALID;
    if (d->kv_format != PA_KV_BF16 && d->kv_format != PA_KV_FP8_E4M3_PAGE_HEAD &&
        d->kv_format != PA_KV_MLA656)
        return PA_ERR_INVALID;
    const int64_t eb = elem_bytes(d->kv_format);
    if ((d->s_page * eb) % 16 || (d->s_head * eb) % 16 || (d->s_tok * eb) % 16) return PA_ERR_INVALID;
    if ((int64_t)d->Hkv * d->G > 65536) return PA_ERR_UNSUPPORTED;
    if (d->q_len > kMaxQLen) return PA_ERR_UNSUPPORTED;
    if (d->window < 0 || d->topk < 0) return PA_ERR_INVALID;
    if (d->topk > 0 && (d->kv_format != PA_KV_MLA656 || d->window > 0 || d->q_len != 1))
        return PA_ERR_UNSUPPORTED;     // sparse decode: MLA tokens, one query token
    if (d->topk > (1 << 24)) return PA_ERR_UNSUPPORTED;
    const int P = d->page_size;
    if (P != 16 && P != 32 && P != 64 && P != 128 && P != 256) return PA_ERR_UNSUPPORTED;
    if (d->B > pa::kMaxBatch) return PA_ERR_UNSUPPORTED;
    if (d->num_splits > 256) return PA_ERR_UNSUPPORTED;
    // fused combine: the merging workgroup reaches a request's partial rows through one
    // buffer with 32-bit byte offsets; a request has at most num_splits chunks (balanced
    // plan: at most kMaxPlanParts)
    if ((d->flags & PA_FLAG_FUSED_COMBINE) &&
        (int64_t)(d->num_splits > 0 ? d->num_splits : pa::kMaxPlanParts) * d->q_len * d->Hkv * d->G * d->Dv * 4 >=
            ((int64_t)1 << 31))
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)d->max_pages_per_seq * P > (int64_t)1 << 30) return PA_ERR_UNSUPPORTED;
    if (d->kv_format == PA_KV_MLA656) {
        // fused combine: one query token (a head group of the MLA kernel is then a range
        // of heads, the unit the in-kernel merge works on), no sparse indices (the sparse
        // variant has no registers to spare for it)
        if ((d->flags & PA_FLAG_FUSED_COMBINE) && (d->q_len != 1 || d->topk > 0))
            return PA_ERR_UNSUPPORTED;
        if (d->Hkv != 1 || d->D != 576 || d->Dv != 512) return PA_ERR_UNSUPPORTED;
        if (d->G % 16 != 0 || d->G > 128) return PA_ERR_UNSUPPORTED;   // 16 heads per wave
        if (d->G * d->q_len > 1024) return PA_ERR_UNSUPPORTED;         // 16 groups of 64 rows
        if (d->s_tok < 656) return PA_ERR_INVALID;
        if (d->s_tok > (1 << 20)) return PA_ERR_UNSUPPORTED;          // 32-bit token offsets
        return PA_OK;
    }
    if (d->D != d->Dv || (d->D != 64 && d->D != 128)) return PA_ERR_UNSUPPORTED;
    if (d->G > 16) return PA_ERR_UNSUPPORTED;
    if (d->G * d->q_len > 256) return PA_ERR_UNSUPPORTED;   // 16 column tiles of 16 rows
    // a token row must fit inside the stride it is read with
    if (d->s_tok < d->D) return PA_ERR_INVALID;
    return PA_OK;
}

// Workgroups along the part axis.  Balanced rule: one workgroup per compute unit over
// all KV heads, so that every unit gets an equal share of each head's tiles.  One
// 4-wave workgroup per unit already keeps enough KV loads in flight to stream at the
// HBM read ceiling; more parts would only cut requests into more chunks to merge.
pa_status num_parts_for(const pa_decode_desc *d, int *np)
{
    if (d->num_splits > 0) {
        *np = d->B * d->num_splits;
        return PA_OK;
    }
    const int cu = cu_count();
    if (cu <= 0) return PA_ERR_DEVICE;
    int n;
    if (d->kv_format == PA_KV_MLA656) {
        // one workgroup per CU over all (part, 64-row group) pairs; rows = G x q_len
        const int ngroups = (d->G * d->q_len + 63) / 64;
        n = cu / ngroups;
    } else {
        const int wgs_per_cu = PA_WGS_PER_CU;
        n = (cu * wgs_per_cu + d->Hkv - 1) / d->Hkv;
    }
    // (the plan kernel keeps the per-part prefix in LDS: at most kMaxPlanParts parts)
    *np = n < 1 ? 1 : (n > pa::kMaxPlanParts ? pa::kMaxPlanParts : n);
    return PA_OK;
}

pa_status layout_for(const pa_decode_desc *d, PlanLayout *L)
{
    int np = 0;
    pa_status st = num_parts_for(d, &np);
    if (st != PA_OK) return st;
    const int rowgroups = d->kv_format == PA_KV_MLA656 ? (d->G * d->q_len + 63) / 64 : d->Hkv;
    *L = pa::plan_layout(d->B, rowgroups, d->num_splits, np);
    return PA_OK;
}

// Device buffer of the no-allocation entry point (plan words, then the partials): one
// copy per device, reserved when the library is loaded there and kept until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is only a
// handle); it uses the device address that hipGetSymbolAddress returns, kept per device.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];
std::atomic<uintptr_t> g_scratch[kMaxDevices];

// Device address of this device's scratch (looked up on the first call on the device).
pa_status scratch_base(uint8_t **base)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_DEVICE;
    uintptr_t v = g_scratch[dev].load(std::memory_order_acquire);
    if (v == 0) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return PA_ERR_DEVICE;
        v = (uintptr_t)ptr;
        g_scratch[dev].store(v, std::memory_order_release);
    }
    *base = (uint8_t *)v;
    return PA_OK;
}

// Pointer and value checks of a decode launch (the desc is already checked).
pa_status check_run_args(const pa_decode_desc *desc, const void *q, const void *k_pool,
                         const void *v_pool, const float *k_scale, const float *v_scale,
                         const int32_t *block_table, const int32_t *seq_lens,
                         const int32_t *indices, const float *sinks, float scale, void *out,
                         float *lse)
{
    if (!q || !k_pool || !block_table || !seq_lens || !out || !lse) return PA_ERR_INVALID;
    if ((desc->topk > 0) != (indices != nullptr)) return PA_ERR_INVALID;
    if (((uintptr_t)indices & 3) || ((uintptr_t)sinks & 3)) return PA_ERR_INVALID;
    const bool fp8 = desc->kv_format == PA_KV_FP8_E4M3_PAGE_HEAD;
    const bool mla = desc->kv_format == PA_KV_MLA656;
    if (mla ? v_pool != nullptr : !v_pool) return PA_ERR_INVALID;
    if (fp8 && (!k_scale || !v_scale)) return PA_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k_pool) || (!mla && !aligned16(v_pool)) || !aligned16(out) ||
        ((uintptr_t)lse & 3) || ((uintptr_t)block_table & 3) || ((uintptr_t)seq_lens & 3))
        return PA_ERR_INVALID;
    if (!isfinite(scale)) return PA_ERR_INVALID;
    return PA_OK;
}

// Enqueue the decode kernel for validated arguments.
pa_status launch_run(const pa_decode_desc *desc, const PlanLayout &L, void *plan, const void *q,
                     const void *k_pool, const void *v_pool, const float *k_scale,
                     const float *v_scale, const int32_t *block_table, const int32_t *seq_lens,
                     const int32_t *indices, const float *sinks, float scale, void *out,
                     float *lse, void *workspace, hipStream_t stream)
{
    pa::DecodeArgs a;
    memset(&a, 0, sizeof a);
    const int64_t eb = elem_bytes(desc->kv_format);
    a.q = (const uint16_t *)q;
    a.k_pool = (const uint8_t *)k_pool;
    a.v_pool = (const uint8_t *)v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table;
    a.plan = (const int32_t *)plan;
    a.out = (uint16_t *)out;
    a.lse = lse;
    a.ws_o = (float *)workspace;
    a.ws_lse = workspace ? (float *)((uint8_t *)workspace +
                                     pa::ws_o_bytes(L.max_items,
                                                    desc->q_len * desc->Hkv * desc->G, desc->Dv))
                         : nullptr;
    a.seq_lens = seq_lens;
    a.indices = indices;
    a.sinks = sinks;
    a.q_len = desc->q_len;
    a.window = desc->window;
    a.topk = desc->topk;
    a.s_page_b = desc->s_page * eb;
    a.s_head_b = desc->s_head * eb;
    a.s_tok_b = desc->s_tok * eb;
    a.B = desc->B;
    a.Hkv = desc->Hkv;
    a.G = desc->G;
    a.D = desc->D;
    a.Dv = desc->Dv;
    a.max_pages = desc->max_pages_per_seq;
    a.page_shift = __builtin_ctz((unsigned)desc->page_size);
    a.num_parts = L.num_parts;
    a.part_begin_off = L.part_begin_off;
    a.items_off = L.items_off;
    a.chunk_off_off = L.chunk_off_off;
    a.fixed_splits = desc->num_splits > 0 ? desc->num_splits : 0;
    a.counters = (desc->flags & PA_FLAG_FUSED_COMBINE) && desc->num_splits != 1
                     ? (int32_t *)plan + L.counters_off
                     : nullptr;
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)desc->D);
    a.scale_log2 = sc * 1.4426950408889634f;
    a.kv_format = desc->kv_format;
    const hipError_t e = desc->kv_format == PA_KV_MLA656 ? pa::launch_mla(a, stream)
                                                         : pa::launch_decode(a, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_DEVICE;
}

// Enqueue the combine kernel (nothing for one chunk per request or a fused run).
pa_status launch_combine_for(const pa_decode_desc *desc, const PlanLayout &L, const void *plan,
                             const void *workspace, const float *sinks, void *out, float *lse,
                             hipStream_t stream)
{
    if (desc->num_splits == 1 || (desc->flags & PA_FLAG_FUSED_COMBINE)) return PA_OK;
    const float *ws_o = (const float *)workspace;
    const float *ws_lse = (const float *)((const uint8_t *)workspace +
                                          pa::ws_o_bytes(L.max_items,
                                                         desc->q_len * desc->Hkv * desc->G,
                                                         desc->Dv));
    if (pa::launch_combine((const int32_t *)plan, ws_o, ws_lse, sinks, (uint16_t *)out, lse, desc->B,
                           desc->Hkv, desc->G, desc->q_len, desc->Dv, L.chunk_off_off,
                           desc->num_splits > 0 ? desc->num_splits : 0, desc->kv_format, stream) != hipSuccess)
        return PA_ERR_DEVICE;
    return PA_OK;
}

}  // namespace

extern "C" {

const char *pa_status_string(int s)
{
    switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or format";
    case PA_ERR_SIZE: return "plan or workspace buffer too small";
    case PA_ERR_DEVICE: return "HIP device error";
    }
    return "unknown status";
}

pa_status pa_kv_append(const pa_decode_desc *desc, int32_t n_new, const void *k_new,
                       const void *v_new, const int32_t *block_table, const int32_t *seq_lens,
                       void *k_pool, void *v_pool, float *k_scale, float *v_scale, void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK) return st;
    if (n_new <= 0) return PA_ERR_INVALID;
    if (n_new > kMaxAppendTokens) return PA_ERR_UNSUPPORTED;
    const bool mla = desc->kv_format == PA_KV_MLA656;
    const bool fp8 = desc->kv_format == PA_KV_FP8_E4M3_PAGE_HEAD;
    if (!k_new || !block_table || !seq_lens || !k_pool) return PA_ERR_INVALID;
    if (mla ? (v_new != nullptr || v_pool != nullptr) : (!v_new || !v_pool)) return PA_ERR_INVALID;
    if (fp8 && (!k_scale || !v_scale)) return PA_ERR_INVALID;
    if (!aligned16(k_new) || !aligned16(k_pool) || (!mla && (!aligned16(v_new) || !aligned16(v_pool))) ||
        ((uintptr_t)block_table & 3) || ((uintptr_t)seq_lens & 3) || ((uintptr_t)k_scale & 3) ||
        ((uintptr_t)v_scale & 3))
        return PA_ERR_INVALID;
    if (pa::launch_append(desc, n_new, k_new, v_new, block_table, seq_lens, k_pool, v_pool,
                          k_scale, v_scale, (hipStream_t)stream) != hipSuccess)
        return PA_ERR_DEVICE;
    return PA_OK;
}

pa_status pa_decode_num_parts(const pa_decode_desc *desc, int32_t *num_parts)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK) return st;
    if (!num_parts) return PA_ERR_INVALID;
    int np = 0;
    st = num_parts_for(desc, &np);
    if (st == PA_OK) *num_parts = np;
    return st;
}

pa_status pa_decode_plan(const pa_decode_desc *desc, const int32_t *seq_lens, void *plan,
                         size_t *plan_bytes, size_t *workspace_bytes, void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK) return st;
    PlanLayout L;
    st = layout_for(desc, &L);
    if (st != PA_OK) return st;
    const size_t pbytes = L.words * 4;
    const size_t wbytes =
        pa::ws_bytes(L.max_items, desc->q_len * desc->Hkv * desc->G, desc->Dv);
    if (!plan) {
        if (plan_bytes) *plan_bytes = pbytes;
        if (workspace_bytes) *workspace_bytes = wbytes;
        return PA_OK;
    }
    if (!seq_lens || !plan_bytes) return PA_ERR_INVALID;
    if (((uintptr_t)plan & 3) || ((uintptr_t)seq_lens & 3)) return PA_ERR_INVALID;
    if (*plan_bytes < pbytes) return PA_ERR_SIZE;
    if (workspace_bytes) *workspace_bytes = wbytes;
    if (pa::launch_plan(seq_lens, (int32_t *)plan, L, desc, (hipStream_t)stream) != hipSuccess)
        return PA_ERR_DEVICE;
    return PA_OK;
}

pa_status pa_decode_run(const pa_decode_desc *desc, void *plan, const void *q,
                        const void *k_pool, const void *v_pool, const float *k_scale,
                        const float *v_scale, const int32_t *block_table,
                        const int32_t *seq_lens, const int32_t *indices, const float *sinks,
                        float scale, void *out, float *lse, void *workspace, void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK) return st;
    if (!plan) return PA_ERR_INVALID;
    st = check_run_args(desc, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, indices,
                        sinks, scale, out, lse);
    if (st != PA_OK) return st;
    if (((uintptr_t)plan & 3)) return PA_ERR_INVALID;
    const bool needs_ws = !(desc->num_splits == 1);
    if (needs_ws && (!workspace || !aligned16(workspace))) return PA_ERR_INVALID;
    PlanLayout L;
    st = layout_for(desc, &L);
    if (st != PA_OK) return st;
    return launch_run(desc, L, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                      indices, sinks, scale, out, lse, workspace, (hipStream_t)stream);
}

pa_status pa_decode_combine(const pa_decode_desc *desc, const void *plan, const void *workspace,
                            const float *sinks, void *out, float *lse, void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK) return st;
    if (!plan || !out || !lse) return PA_ERR_INVALID;
    if (desc->num_splits == 1) return PA_OK;     // every request is a single chunk
    if (desc->flags & PA_FLAG_FUSED_COMBINE) return PA_OK;   // pa_decode_run merged
    if (!workspace || !aligned16(workspace) || !aligned16(out) || ((uintptr_t)lse & 3) ||
        ((uintptr_t)sinks & 3))
        return PA_ERR_INVALID;
    PlanLayout L;
    st = layout_for(desc, &L);
    if (st != PA_OK) return st;
    return launch_combine_for(desc, L, plan, workspace, sinks, out, lse, (hipStream_t)stream);
}

pa_status pa_decode_noalloc(const pa_decode_desc *desc, const void *q, const void *k_pool,
                            const void *v_pool, const float *k_scale, const float *v_scale,
                            const int32_t *block_table, const int32_t *seq_lens,
                            const int32_t *indices, const float *sinks, float scale, void *out,
                            float *lse, void *stream)
{
    pa_status st = check_desc(desc);
    if (st != PA_OK) return st;
    st = check_run_args(desc, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, indices,
                        sinks, scale, out, lse);
    if (st != PA_OK) return st;
    PlanLayout L;
    st = layout_for(desc, &L);
    if (st != PA_OK) return st;
    const size_t plan_bytes = (L.words * 4 + 255) & ~(size_t)255;
    const size_t ws = pa::ws_bytes(L.max_items, desc->q_len * desc->Hkv * desc->G, desc->Dv);
    if (plan_bytes + ws > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SIZE;
    uint8_t *base = nullptr;
    st = scratch_base(&base);
    if (st != PA_OK) return st;
    void *plan = base, *workspace = base + plan_bytes;
    const hipStream_t s = (hipStream_t)stream;
    if (pa::launch_plan(seq_lens, (int32_t *)plan, L, desc, s) != hipSuccess) return PA_ERR_DEVICE;
    st = launch_run(desc, L, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                    indices, sinks, scale, out, lse, workspace, s);
    if (st != PA_OK) return st;
    return launch_combine_for(desc, L, plan, workspace, sinks, out, lse, s);
}

}  // extern "C"
