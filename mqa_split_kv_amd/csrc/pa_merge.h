// Device-side LSE merge of chunk partials, used by the combine kernel and by the
// fused-combine epilogue of the decode kernels (the last workgroup to finish a
// request's chunks merges them).  XQA article, section "归约怎么记", merge equation,
// written for normalised partials O_i with natural-log lse_i:
//   M = max_i lse_i,  lse = M + ln sum_i exp(lse_i - M),  out = sum_i exp(lse_i - lse) O_i.
// Chunks with lse_i = -inf (empty ranges) carry no weight; rows with no non-empty chunk
// get out = 0 and lse = -inf, without forming -inf - (-inf) (pipelining page, section 三).
#pragma once

#include "pa_internal.h"

// The fused combine's ordering (relaxed agent-scope atomics plus a wait for the stores,
// below) relies on gfx950's cross-XCD coherence of agent-scope accesses; no other device
// target is built.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "pa_merge.h: the fused-combine ordering is written for gfx950 only"
#endif

namespace pa {

typedef __bf16 merge_bf16x4 __attribute__((ext_vector_type(4)));
typedef float merge_f32x4 __attribute__((ext_vector_type(4)));

// Query row qr = qi * Hq + hq (query token qi, head hq; nq tokens per request).  Its
// partial in chunk c is ws_o[(c * nq * Hq + qr) * Dv ...], ws_lse[c * nq * Hq + qr]; its
// output out[(b * nq * Hq + qr) * Dv ...], lse[b * nq * Hq + qr].  Merges heads
// [hq0, hq0 + nrows) of every query token of request b from chunks c0 .. c0 + n - 1.  A
// work unit is one (query token, head) row and 4 dims; thread tid takes units tid, tid + nthr, ... kUnits at a
// time (1 in the wide combine grid, 1 to 4 in a single fused-combine workgroup), and reads the
// chunks kBatch at a time with a running maximum (the same rescaling as the online
// softmax), so that up to kUnits x kBatch partial loads are in flight instead of one
// dependent load after another.  A unit's arithmetic does not depend on kUnits, and both
// callers take the batch from merge_batch(), so both produce the same bits.  The result is
//   out = sum_i exp(lse_i - M) O_i / sum_i exp(lse_i - M),  lse = M + ln sum_i exp(lse_i - M)
// which is the merge equation above with exp(lse_i - lse) = exp(lse_i - M) / sum.  An
// attention sink (sinks[hq], natural-log units, or null) joins once as one more partial
// with lse = sink and O = 0 (XQA article, section "一个容易漏掉的细节: attention sink":
// the final reduction adds the sink to the denominator).
// Chunks per load round: 8 when requests are cut into many chunks (fixed splits, the
// bf16 / fp8 balanced plans), 4 for the MLA workload's 2-3 chunks per request, where 8
// mostly issues masked loads (measured on MI355X: combine kernel 11.3 against 12.8 us on the
// MLA workload).
__host__ __device__ inline int merge_batch(int kv_format) { return kv_format == PA_KV_MLA656 ? 4 : 8; }

// Partials shared across workgroups inside one launch (the fused combine) are written and
// read with the cache policy of agent-scope relaxed atomics: on gfx950 such stores and
// loads (single floats here, 16 bytes through the buffer helpers below) are coherent at
// device scope by themselves (the sc1 cache policy: through the non-coherent per-XCD L2),
// so ordering them only takes a wait for the stores and the counter atomic, and no fence,
// i.e. no write-back or invalidation of the whole L2.
__device__ inline void store_shared(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_shared(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same cache policy (sc1) on 16-byte accesses, through a buffer over a uniform range of
// partial rows (one item's or one request's, far below 2^32 bytes): a quarter of the
// memory instructions of four single-float accesses.  `base` must be uniform.
__device__ inline __amdgpu_buffer_rsrc_t shared_rows(const float *base, int64_t nbytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)nbytes, 0x00020000);
}
constexpr int kCoherentPolicy = 16;     // the sc1 bit of the buffer instructions' cache policy
__device__ inline merge_f32x4 load_shared4(__amdgpu_buffer_rsrc_t rows, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rows, byte_off, 0, kCoherentPolicy);
}
__device__ inline void store_shared4(__amdgpu_buffer_rsrc_t rows, uint32_t byte_off, merge_f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, rows, byte_off, 0, kCoherentPolicy);
}

// COHERENT: the partials come from other workgroups of the same launch (read with
// load_shared); else from an earlier launch (plain loads).
template <int kUnits, bool COHERENT, int kBatch>
__device__ inline void merge_rows_b(const float *ws_o, const float *ws_lse, const float *sinks,
                                  uint16_t *out, float *lse, int b, int64_t c0, int n, int Hq,
                                  int nq, int Dv, int hq0, int nrows, int tid, int nthr)
{
    const int q4 = Dv / 4;
    const int total = nq * nrows * q4;
    const int64_t Hr = (int64_t)nq * Hq;                 // query rows per request / chunk
    // COHERENT: the request's n chunks of partial rows, read 16 bytes at a time
    const __amdgpu_buffer_rsrc_t rows_o = shared_rows(ws_o + c0 * Hr * Dv, COHERENT ? (int64_t)n * Hr * Dv * 4 : 0);
    auto qrow = [&](int u) {
        const int rr = u / q4;
        return (rr / nrows) * Hq + hq0 + rr % nrows;
    };
    for (int u0 = tid; u0 < total; u0 += kUnits * nthr) {
        int64_t prow0[kUnits];
        bool ok[kUnits];
        float m[kUnits], s[kUnits];
        merge_f32x4 acc[kUnits];
#pragma unroll
        for (int j = 0; j < kUnits; j++) {
            const int u = u0 + j * nthr;
            ok[j] = u < total;
            prow0[j] = c0 * Hr + qrow(ok[j] ? u : 0);
            m[j] = -INFINITY;
            s[j] = 0.f;
            if (sinks && ok[j]) {
                m[j] = sinks[hq0 + (u / q4) % nrows];   // the sink's partial: (sink, 1, 0)
                s[j] = 1.f;
            }
            acc[j] = merge_f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int i0 = 0; i0 < n; i0 += kBatch) {
            float lv[kUnits][kBatch];
            merge_f32x4 ov[kUnits][kBatch];
#pragma unroll
            for (int j = 0; j < kUnits; j++) {
                const int d0 = ((u0 + j * nthr) % q4) * 4;
#pragma unroll
                for (int k = 0; k < kBatch; k++) {
                    const bool in = ok[j] && i0 + k < n;
                    const int64_t prow = prow0[j] + (int64_t)(i0 + k) * Hr;
                    if (COHERENT) {
                        lv[j][k] = in ? load_shared(ws_lse + prow) : -INFINITY;
                        ov[j][k] = in ? load_shared4(rows_o, (uint32_t)(((prow - c0 * Hr) * Dv + d0) * 4))
                                      : merge_f32x4{0.f, 0.f, 0.f, 0.f};
                    } else {
                        lv[j][k] = in ? ws_lse[prow] : -INFINITY;
                        ov[j][k] = in ? *(const merge_f32x4 *)(ws_o + prow * Dv + d0)
                                      : merge_f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kUnits; j++) {
                float mb = m[j];
#pragma unroll
                for (int k = 0; k < kBatch; k++) mb = fmaxf(mb, lv[j][k]);
                if (mb == -INFINITY) continue;            // nothing non-empty yet
                const float alpha = expf(m[j] - mb);      // m = -inf: 0
                s[j] *= alpha;
                acc[j] *= alpha;
#pragma unroll
                for (int k = 0; k < kBatch; k++) {
                    if (lv[j][k] == -INFINITY) continue;  // empty chunk: no weight
                    const float w = expf(lv[j][k] - mb);
                    s[j] += w;
                    acc[j] += w * ov[j][k];
                }
                m[j] = mb;
            }
        }
#pragma unroll
        for (int j = 0; j < kUnits; j++) {
            if (!ok[j]) continue;
            const int u = u0 + j * nthr;
            const int d0 = (u % q4) * 4;
            const int64_t row = (int64_t)b * Hr + qrow(u);
            merge_bf16x4 ob;
            if (m[j] == -INFINITY) {
                ob = merge_bf16x4{};
                if (d0 == 0) lse[row] = -INFINITY;
            } else {
                const float inv = 1.0f / s[j];
#pragma unroll
                for (int k = 0; k < 4; k++) ob[k] = (__bf16)(acc[j][k] * inv);
                if (d0 == 0) lse[row] = m[j] + logf(s[j]);
            }
            *(merge_bf16x4 *)(out + row * Dv + d0) = ob;
        }
    }
}

// merge_rows_b with the batch chosen at run time (merge_batch)
template <int kUnits, bool COHERENT = false>
__device__ inline void merge_rows(int batch, const float *ws_o, const float *ws_lse, const float *sinks,
                                  uint16_t *out, float *lse, int b, int64_t c0, int n, int Hq,
                                  int nq, int Dv, int hq0, int nrows, int tid, int nthr)
{
    if (batch == 4)
        merge_rows_b<kUnits, COHERENT, 4>(ws_o, ws_lse, sinks, out, lse, b, c0, n, Hq, nq, Dv, hq0, nrows, tid, nthr);
    else
        merge_rows_b<kUnits, COHERENT, 8>(ws_o, ws_lse, sinks, out, lse, b, c0, n, Hq, nq, Dv, hq0, nrows, tid, nthr);
}

// Fused combine, called by every thread of a workgroup once it has processed all its
// items [ib, ie) (kUnits: the merge's units per thread and pass, as in merge_rows) (row group rg: query heads [hq0, hq0 + nrows) of every query token;
// `arrivals` workgroups write partials per chunk of the row group).  The partials were
// written with store_shared / store_shared4; each thread waits until its stores are complete, the
// workgroup meets, and one thread counts each of the workgroup's partial chunks in with a
// device-scope atomic; the workgroup that counts a request's last chunk reads the other
// workgroups' partials with load_shared / load_shared4 (every store it needs completed before the count
// it observed), merges that request, and returns its counter to zero.  Then requests with no chunk at all (length 0 under the
// balanced rule) get out = 0, lse = -inf (or the sink) from workgroup part = b mod
// num_parts.
template <int kUnits = 4>
__device__ inline void fused_combine_tail(const DecodeArgs &a, const int32_t *plan, int part,
                                          int ib, int ie, int rg, int n_rowgroups, int hq0,
                                          int nrows, int arrivals, int *s_flag)
{
    const int Hq = a.Hkv * a.G, nq = a.q_len;
    // with every request in one chunk the fused path costs nothing
    bool wrote = false;
    for (int it = ib; it < ie; it++) wrote |= !(plan[a.items_off + 4 * it + 3] & 1);
    if (wrote) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's partials are out
        __syncthreads();
    }
    for (int it = ib; it < ie; it++) {
        if (plan[a.items_off + 4 * it + 3] & 1) continue;   // single chunk: already final
        const int b = plan[a.items_off + 4 * it + 0];
        const int c0 = plan[a.chunk_off_off + b];
        const int n = plan[a.chunk_off_off + b + 1] - c0;
        int32_t *cnt = a.counters + (int64_t)b * n_rowgroups + rg;
        if (threadIdx.x == 0)
            *s_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      n * arrivals - 1;
        __syncthreads();
        if (*s_flag) {
            merge_rows<kUnits, true>(merge_batch(a.kv_format), a.ws_o, a.ws_lse, a.sinks, a.out, a.lse, b, c0,
                                     n, Hq, nq, a.Dv, hq0, nrows, threadIdx.x, blockDim.x);
            if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    }
    for (int b = part; b < a.B; b += a.num_parts) {
        if (plan[a.chunk_off_off + b + 1] != plan[a.chunk_off_off + b]) continue;
        const int q4 = a.Dv / 4;
        for (int u = threadIdx.x; u < nq * nrows * q4; u += blockDim.x) {
            const int rr = u / q4, d0 = (u % q4) * 4;
            const int64_t row = ((int64_t)b * nq + rr / nrows) * Hq + hq0 + rr % nrows;
            *(merge_bf16x4 *)(a.out + row * a.Dv + d0) = merge_bf16x4{};
            if (d0 == 0) a.lse[row] = a.sinks ? a.sinks[hq0 + rr % nrows] : -INFINITY;
        }
    }
}

}  // namespace pa
