// Combine kernel: LSE-weighted merge of the per-chunk partials of every request that
// the plan cut into several chunks, and out = 0 / lse = -inf for requests with no
// chunk (XQA article, section "归约怎么记", merge equation; FlashMLA walk-through,
// section 合并与性能账本: partials carry o and lse).  The arithmetic is merge_rows.
#include "pa_merge.h"

namespace pa {
namespace {

// one wave per workgroup: a (request, KV head)'s rows spread over several small workgroups,
// every lane busy (HD64: 128 units of 4 dims per (request, head) -> 2 workgroups), so that
// the partial loads of all of them are in flight on more compute units at once
constexpr int kCombineThreads = 64;

__global__ __launch_bounds__(kCombineThreads) void pa_combine_kernel(
    const int32_t *__restrict__ plan, const float *__restrict__ ws_o,
    const float *__restrict__ ws_lse, const float *__restrict__ sinks, uint16_t *__restrict__ out,
    float *__restrict__ lse, int Hkv, int G, int q_len, int Dv, int chunk_off_off, int fixed_splits,
    int batch)
{
    const int bh = blockIdx.x;
    const int b = bh / Hkv, h = bh % Hkv;
    // a fixed-split plan cuts every request into the same count (no plan read needed)
    const int c0 = fixed_splits > 0 ? b * fixed_splits : plan[chunk_off_off + b];
    const int n = fixed_splits > 0 ? fixed_splits : plan[chunk_off_off + b + 1] - c0;
    if (n == 1) return;                           // the decode kernel wrote this row
    merge_rows<1>(batch, ws_o, ws_lse, sinks, out, lse, b, c0, n, Hkv * G, q_len, Dv, h * G, G,
                  blockIdx.y * kCombineThreads + threadIdx.x, gridDim.y * kCombineThreads);
}

}  // namespace

hipError_t launch_combine(const int32_t *plan, const float *ws_o, const float *ws_lse,
                          const float *sinks, uint16_t *out, float *lse, int B, int Hkv, int G,
                          int q_len, int Dv, int chunk_off_off, int fixed_splits, int kv_format,
                          hipStream_t stream)
{
    const int per_bh = q_len * G * (Dv / 4);
    const dim3 grid(B * Hkv, (per_bh + kCombineThreads - 1) / kCombineThreads);
    hipLaunchKernelGGL(pa_combine_kernel, grid, dim3(kCombineThreads), 0, stream, plan, ws_o,
                       ws_lse, sinks, out, lse, Hkv, G, q_len, Dv, chunk_off_off, fixed_splits,
                       merge_batch(kv_format));
    return hipGetLastError();
}

}  // namespace pa
