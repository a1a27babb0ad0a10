// KV append: writes the new tokens' K/V into their pages before attention reads them
// (XQA article, section "一次 decode step 的完整时序": the step's K/V are in the paged
// cache before the attention kernel runs).  New token j of request b goes to position
// seq_lens[b] - n_new + j (seq_lens are the lengths after the append).
//
//  * bf16 pools: a scatter of 16-byte chunks.
//  * fp8 page-head pools: the (page, KV head) scale is the running max|x| / 448 of what
//    the page has received.  Per page that gets new tokens (slots [s0, s1)), in position
//    order: amax over the new values; a fresh page (s0 = 0) takes amax / 448 (1 if
//    amax = 0); otherwise scale = max(old, amax / 448) and, when it grows, the page's
//    older codes are re-encoded as e4m3(fp32(fp32(decode(c) * old) / scale)); new codes
//    are e4m3(fp32(x / scale)).  K and V have their own scales (grid z).
//  * MLA 656-byte tokens (FlashMLA walk-through, section 数据加载): per token and
//    128-value tile, scale = max|x| / 448 (1 if 0), codes e4m3(fp32(x / scale)), the 64
//    rope values copied.
// e4m3 is OCP E4M3FN, round to nearest even, magnitudes beyond 448 saturate.
// A workgroup owns the pages it writes: pages that receive new tokens must belong to
// one request.
#include "pa_internal.h"

namespace pa {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 256;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> e4m3 code, round to nearest even (gfx950 conversion), saturating at +-448, NaN
// to 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float x)
{
    if (x != x) return 0x7Fu;
    const float c = fminf(fmaxf(x, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xFFu;
}

// the 4 e4m3 codes of a word -> fp32 (exact)
__device__ __forceinline__ void e4m3x4_values(uint32_t word, float v[4])
{
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
    v[0] = lo[0];
    v[1] = lo[1];
    v[2] = hi[0];
    v[3] = hi[1];
}

// max over the workgroup (all threads call; result in every thread)
__device__ float block_max(float v, float *s_red)
{
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s_red[w] = v;
    __syncthreads();
    float r = s_red[0];
    for (int i = 1; i < kAppendThreads / 64; i++) r = fmaxf(r, s_red[i]);
    __syncthreads();
    return r;
}

struct AppendArgs {
    const uint16_t *k_new, *v_new;      // [B][n_new][Hkv][D] bf16 (MLA: [B][n_new][576])
    const int32_t *block_table, *seq_lens;
    uint8_t *k_pool, *v_pool;
    float *k_scale, *v_scale;
    int64_t s_page_b, s_head_b, s_tok_b;
    int B, Hkv, D, page_size, max_pages, n_new;
};

// bf16: grid (B, Hkv), every new token row of K and V copied in 16-byte chunks
__global__ __launch_bounds__(kAppendThreads) void pa_append_bf16_kernel(AppendArgs a)
{
    const int b = blockIdx.x, h = blockIdx.y;
    const int L = a.seq_lens[b];
    const int cpr = a.D * 2 / 16;                    // chunks per token row
    for (int u = threadIdx.x; u < 2 * a.n_new * cpr; u += kAppendThreads) {
        const int which = u / (a.n_new * cpr);
        const int j = (u / cpr) % a.n_new, c = u % cpr;
        const int pos = L - a.n_new + j;
        if (pos < 0) continue;
        const int64_t page = a.block_table[(int64_t)b * a.max_pages + pos / a.page_size];
        const int64_t dst = page * a.s_page_b + (int64_t)h * a.s_head_b +
                            (int64_t)(pos % a.page_size) * a.s_tok_b + 16 * c;
        const uint16_t *src = (which ? a.v_new : a.k_new) + (((int64_t)b * a.n_new + j) * a.Hkv + h) * a.D;
        *(u32x4 *)((which ? a.v_pool : a.k_pool) + dst) = *(const u32x4 *)((const uint8_t *)src + 16 * c);
    }
}

// fp8 page-head: grid (B, Hkv, 2): z = 0 appends to the K pool, z = 1 to the V pool
__global__ __launch_bounds__(kAppendThreads) void pa_append_fp8_kernel(AppendArgs a)
{
    __shared__ float s_red[kAppendThreads / 64];
    const int b = blockIdx.x, h = blockIdx.y;
    const bool isv = blockIdx.z != 0;
    const uint16_t *xn = isv ? a.v_new : a.k_new;
    uint8_t *pool = isv ? a.v_pool : a.k_pool;
    float *scales = isv ? a.v_scale : a.k_scale;
    const int L = a.seq_lens[b], P = a.page_size, D = a.D, n_new = a.n_new;
    const int first = L - n_new;
    if (first < 0) return;
    const int wpr = D / 4;                           // 4-code words per token row
    int j = 0;
    while (j < n_new) {
        const int pos0 = first + j;
        const int lp = pos0 / P, s0 = pos0 % P;
        const int cnt = min(n_new - j, P - s0);      // new tokens landing in this page
        const int64_t page = a.block_table[(int64_t)b * a.max_pages + lp];
        uint8_t *pbase = pool + page * a.s_page_b + (int64_t)h * a.s_head_b;
        auto xval = [&](int t, int i) {
            return bf16_bits_to_f32(xn[(((int64_t)b * n_new + j + t) * a.Hkv + h) * D + i]);
        };
        float amax = 0.f;
        for (int u = threadIdx.x; u < cnt * D; u += kAppendThreads) amax = fmaxf(amax, fabsf(xval(u / D, u % D)));
        amax = block_max(amax, s_red);
        float scale;
        if (s0 == 0) {
            scale = amax > 0.f ? amax / 448.0f : 1.0f;
        } else {
            const float old = scales[page * a.Hkv + h];
            const float grown = amax / 448.0f;
            scale = grown > old ? grown : old;
            if (scale > old) {
                // re-encode the page's older codes with the grown scale
                for (int u = threadIdx.x; u < s0 * wpr; u += kAppendThreads) {
                    uint32_t *w = (uint32_t *)(pbase + (int64_t)(u / wpr) * a.s_tok_b) + u % wpr;
                    float v[4];
                    e4m3x4_values(*w, v);
                    uint32_t o = 0;
#pragma unroll
                    for (int k = 0; k < 4; k++) o |= e4m3_code(v[k] * old / scale) << (8 * k);
                    *w = o;
                }
            }
        }
        for (int u = threadIdx.x; u < cnt * wpr; u += kAppendThreads) {
            const int t = u / wpr, i0 = (u % wpr) * 4;
            uint32_t o = 0;
#pragma unroll
            for (int k = 0; k < 4; k++) o |= e4m3_code(xval(t, i0 + k) / scale) << (8 * k);
            *((uint32_t *)(pbase + (int64_t)(s0 + t) * a.s_tok_b) + u % wpr) = o;
        }
        __syncthreads();                             // every thread has read the old scale
        if (threadIdx.x == 0) scales[page * a.Hkv + h] = scale;
        j += cnt;
    }
}

// MLA-656: grid (B, n_new); wave w quantises latent tile w (128 values, 2 per lane)
__global__ __launch_bounds__(kAppendThreads) void pa_append_mla_kernel(AppendArgs a)
{
    const int b = blockIdx.x, j = blockIdx.y;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int pos = a.seq_lens[b] - a.n_new + j;
    if (pos < 0) return;
    const int64_t page = a.block_table[(int64_t)b * a.max_pages + pos / a.page_size];
    uint8_t *tok = a.k_pool + page * a.s_page_b + (int64_t)(pos % a.page_size) * a.s_tok_b;
    const uint16_t *x = a.k_new + ((int64_t)b * a.n_new + j) * 576;
    const uint32_t xx = *(const uint32_t *)(x + 128 * w + 2 * lane);
    const float x0 = bf16_bits_to_f32(xx & 0xFFFFu), x1 = bf16_bits_to_f32(xx >> 16);
    float amax = fmaxf(fabsf(x0), fabsf(x1));
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    const uint32_t codes = e4m3_code(x0 / scale) | (e4m3_code(x1 / scale) << 8);
    *(uint16_t *)(tok + 128 * w + 2 * lane) = (uint16_t)codes;
    if (lane == 0) *(float *)(tok + 512 + 4 * w) = scale;
    if (w == 0 && lane < 32)                          // rope: 64 bf16 = 32 words
        *(uint32_t *)(tok + 528 + 4 * lane) = *(const uint32_t *)(x + 512 + 2 * lane);
}

}  // namespace

hipError_t launch_append(const pa_decode_desc *d, int n_new, const void *k_new, const void *v_new,
                         const int32_t *block_table, const int32_t *seq_lens, void *k_pool,
                         void *v_pool, float *k_scale, float *v_scale, hipStream_t stream)
{
    AppendArgs a;
    const int64_t eb = d->kv_format == PA_KV_BF16 ? 2 : 1;
    a.k_new = (const uint16_t *)k_new;
    a.v_new = (const uint16_t *)v_new;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.k_pool = (uint8_t *)k_pool;
    a.v_pool = (uint8_t *)v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.s_page_b = d->s_page * eb;
    a.s_head_b = d->s_head * eb;
    a.s_tok_b = d->s_tok * eb;
    a.B = d->B;
    a.Hkv = d->Hkv;
    a.D = d->D;
    a.page_size = d->page_size;
    a.max_pages = d->max_pages_per_seq;
    a.n_new = n_new;
    if (d->kv_format == PA_KV_BF16)
        hipLaunchKernelGGL(pa_append_bf16_kernel, dim3(d->B, d->Hkv), dim3(kAppendThreads), 0,
                           stream, a);
    else if (d->kv_format == PA_KV_FP8_E4M3_PAGE_HEAD)
        hipLaunchKernelGGL(pa_append_fp8_kernel, dim3(d->B, d->Hkv, 2), dim3(kAppendThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(pa_append_mla_kernel, dim3(d->B, n_new), dim3(kAppendThreads), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace pa
