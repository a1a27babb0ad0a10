// Combine kernel: LSE-weighted merge of the per-chunk partials of every request that
// the plan cut into several chunks (XQA article, section "归约怎么记", merge
// equation; FlashMLA walk-through, section 合并与性能账本: partials carry o and lse).
// With normalised partials O_i and lse_i:
//   M = max_i lse_i,  lse = M + ln sum_i exp(lse_i - M),  out = sum_i exp(lse_i - lse) O_i.
// Chunks with lse_i = -inf (empty ranges) carry no weight; a request with no
// non-empty chunk (length 0) gets out = 0, lse = -inf without forming -inf - (-inf)
// (pipelining page, section 三, "分数可以早算").
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void pa_combine_kernel(
    const int32_t *__restrict__ plan, const float *__restrict__ ws_o,
    const float *__restrict__ ws_lse, uint16_t *__restrict__ out, float *__restrict__ lse,
    int Hkv, int G, int Dv, int chunk_off_off)
{
    const int bh = blockIdx.x;
    const int b = bh / Hkv, h = bh % Hkv;
    const int c0 = plan[chunk_off_off + b];
    const int n = plan[chunk_off_off + b + 1] - c0;
    if (n == 1) return;                           // the decode kernel wrote this row
    const int idx = blockIdx.y * kCombineThreads + threadIdx.x;
    const int q4 = Dv / 4;
    const int g = idx / q4, d0 = (idx % q4) * 4;
    if (g >= G) return;
    const int Hq = Hkv * G;
    const int64_t row = (int64_t)b * Hq + (int64_t)h * G + g;
    const int64_t stride = (int64_t)Hkv * G;      // partial rows per chunk
    const int64_t prow0 = (int64_t)c0 * stride + (int64_t)h * G + g;

    float M = -INFINITY;
    for (int i = 0; i < n; i++) M = fmaxf(M, ws_lse[prow0 + i * stride]);
    if (M == -INFINITY) {
        *(bf16x4 *)(out + row * Dv + d0) = bf16x4{};
        if (d0 == 0) lse[row] = -INFINITY;
        return;
    }
    float wsum = 0.f;
    for (int i = 0; i < n; i++) {
        const float li = ws_lse[prow0 + i * stride];
        if (li != -INFINITY) wsum += expf(li - M);
    }
    const float lse_tot = M + logf(wsum);
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n; i++) {
        const float li = ws_lse[prow0 + i * stride];
        if (li == -INFINITY) continue;
        const float w = expf(li - lse_tot);
        const f32x4 oi = *(const f32x4 *)(ws_o + (prow0 + i * stride) * Dv + d0);
        o += w * oi;
    }
    bf16x4 ob;
#pragma unroll
    for (int k = 0; k < 4; k++) ob[k] = (__bf16)o[k];
    *(bf16x4 *)(out + row * Dv + d0) = ob;
    if (d0 == 0) lse[row] = lse_tot;
}

}  // namespace

hipError_t launch_combine(const int32_t *plan, const float *ws_o, const float *ws_lse,
                          uint16_t *out, float *lse, int B, int Hkv, int G, int Dv,
                          int chunk_off_off, hipStream_t stream)
{
    const int per_bh = G * (Dv / 4);
    const dim3 grid(B * Hkv, (per_bh + kCombineThreads - 1) / kCombineThreads);
    hipLaunchKernelGGL(pa_combine_kernel, grid, dim3(kCombineThreads), 0, stream, plan, ws_o,
                       ws_lse, out, lse, Hkv, G, Dv, chunk_off_off);
    return hipGetLastError();
}

}  // namespace pa
