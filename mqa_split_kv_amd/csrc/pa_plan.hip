// Split scheduler (plan kernel).
//
// One workgroup reads seq_lens and writes the plan: which (request, token range)
// items each part processes.  Two rules:
//  * fixed: request b is cut into s chunks of ceil(n_b / s) 64-token tiles
//    (FlashAttention tiling page, section 5.3 "Split 在 block.h 中的实现");
//  * balanced: all requests' tiles laid end to end and cut into num_parts equal
//    contiguous parts (FlashMLA walk-through, section 调度: work is shared out over
//    the compute units ahead of the main kernel, equal per unit, and the result can
//    be reused while shapes and lengths stay the same).
// The tiles of request b cover keys [64 * first_b, len_b): len_b = L_b (topk index slots
// for sparse decode) and first_b the tile of the earliest key a sliding window leaves
// visible (XQA article, section "分页 KV: 页号怎么变成 TMA 坐标": leading pages outside
// the window are never read), 0 otherwise.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

struct Span {
    int q_len, window, topk;
    // keys (or index slots) the request's items cover: [64 * first(L), len(L))
    __device__ int len(int L) const { return topk > 0 ? topk : L; }
    __device__ int first(int L) const
    {
        if (topk > 0 || window <= 0) return 0;
        const int lo = L - q_len - window + 1;
        return lo > 0 ? lo / kTileTokens : 0;
    }
    __device__ int tiles(int L) const { return ceil_div_i(len(L), kTileTokens) - first(L); }
};

// Exclusive scan of `n` ints in LDS (in place), returns the total.  All threads call.
__device__ int block_exclusive_scan(int *v, int n, int *scratch)
{
    const int tid = threadIdx.x;
    const int per = ceil_div_i(n, kPlanThreads);
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int s = 0;
    for (int i = lo; i < hi; i++) s += v[i];
    scratch[tid] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan over the per-thread sums
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        int x = tid >= off ? scratch[tid - off] : 0;
        __syncthreads();
        scratch[tid] += x;
        __syncthreads();
    }
    int run = scratch[tid] - s;
    for (int i = lo; i < hi; i++) {
        int x = v[i];
        v[i] = run;
        run += x;
    }
    __syncthreads();
    int total = scratch[kPlanThreads - 1];
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(kPlanThreads) void pa_plan_kernel(
    const int32_t *__restrict__ seq_lens, int32_t *__restrict__ plan, int B, int num_parts,
    int max_items, int num_splits, int part_begin_off, int chunk_off_off, int items_off,
    int counters_off, int n_counters, Span sp)
{
    __shared__ int s_start[kMaxBatch + 1];   // tile prefix S_b
    __shared__ int s_ne[kMaxBatch + 1];      // non-empty request prefix
    __shared__ int s_scratch[kPlanThreads];
    const int tid = threadIdx.x;
    int32_t *part_begin = plan + part_begin_off;
    int32_t *chunk_off = plan + chunk_off_off;
    int32_t *items = plan + items_off;
    // fused-combine counters start at zero (each fused run leaves them at zero again)
    for (int i = tid; i < n_counters; i += kPlanThreads) plan[counters_off + i] = 0;

    if (num_splits > 0) {
        // ---- fixed split count: item p = (b = p / s, i = p % s), one per part
        const int s = num_splits;
        const int n_items = B * s;
        for (int p = tid; p < n_items; p += kPlanThreads) {
            const int b = p / s, i = p % s;
            const int L = sp.len(seq_lens[b]), f = sp.first(seq_lens[b]);
            const int n = sp.tiles(seq_lens[b]);
            const int per = ceil_div_i(n, s);
            const int lo = f + i * per;
            const int hi = f + min((i + 1) * per, n);
            const int t0 = min(lo * kTileTokens, L);
            int t1 = min(hi * kTileTokens, L);
            if (t1 < t0) t1 = t0;
            items[4 * p + 0] = b;
            items[4 * p + 1] = t0;
            items[4 * p + 2] = t1;
            items[4 * p + 3] = s == 1 ? 1 : 0;
        }
        for (int p = tid; p <= n_items; p += kPlanThreads) part_begin[p] = p;
        for (int b = tid; b <= B; b += kPlanThreads) chunk_off[b] = b * s;
        if (tid == 0) {
            plan[0] = kPlanMagic; plan[1] = 0; plan[2] = B; plan[3] = n_items;
            plan[4] = n_items; plan[5] = kTileTokens; plan[6] = max_items; plan[7] = 0;
        }
        return;
    }

    // ---- balanced parts
    for (int b = tid; b < B; b += kPlanThreads) {
        const int n = sp.tiles(seq_lens[b]);
        s_start[b] = n;
        s_ne[b] = n > 0 ? 1 : 0;
    }
    __syncthreads();
    const int N = block_exclusive_scan(s_start, B, s_scratch);
    const int NE = block_exclusive_scan(s_ne, B, s_scratch);
    if (tid == 0) { s_start[B] = N; s_ne[B] = NE; }
    __syncthreads();

    const int64_t Np = num_parts;
    // first tile of part p
    auto edge = [&](int p) -> int { return (int)(((int64_t)p * N) / Np); };
    // part containing global tile x (0 <= x < N): largest p with edge(p) <= x
    auto part_of = [&](int x) -> int { return (int)((((int64_t)x + 1) * Np - 1) / N); };
    // request containing global tile x: largest b with S_b <= x (it is non-empty)
    auto req_of = [&](int x) -> int {
        int lo = 0, hi = B;                  // S_lo <= x < S_hi
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if (s_start[mid] <= x) lo = mid; else hi = mid;
        }
        return lo;
    };

    // items per part -> part_begin (exclusive scan over parts, in global memory)
    // parts are processed in strided chunks; the count is kept in part_begin first.
    for (int p = tid; p < num_parts; p += kPlanThreads) {
        const int e0 = edge(p), e1 = edge(p + 1);
        int cnt = 0;
        if (e1 > e0) {
            const int bf = req_of(e0), bl = req_of(e1 - 1);
            cnt = s_ne[bl + 1] - s_ne[bf];
        }
        part_begin[p] = cnt;
    }
    __threadfence_block();
    __syncthreads();
    // exclusive scan of part_begin[0..num_parts) in global memory, by the whole block
    {
        const int per = ceil_div_i(num_parts, kPlanThreads);
        const int lo = min(num_parts, tid * per), hi = min(num_parts, lo + per);
        int s = 0;
        for (int i = lo; i < hi; i++) s += part_begin[i];
        s_scratch[tid] = s;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            int x = tid >= off ? s_scratch[tid - off] : 0;
            __syncthreads();
            s_scratch[tid] += x;
            __syncthreads();
        }
        int run = s_scratch[tid] - s;
        for (int i = lo; i < hi; i++) {
            int x = part_begin[i];
            part_begin[i] = run;
            run += x;
        }
        if (tid == 0) part_begin[num_parts] = s_scratch[kPlanThreads - 1];
    }
    __threadfence_block();
    __syncthreads();

    // chunks per request -> chunk_off
    for (int b = tid; b < B; b += kPlanThreads) {
        const int n = s_start[b + 1] - s_start[b];
        // When N >= num_parts every part holds at least one tile, so the parts a request
        // touches are consecutive and all non-empty.  Otherwise every non-empty part holds
        // exactly one tile and the request has one chunk per tile.
        int nch = 0;
        if (n > 0)
            nch = (int64_t)N >= Np ? part_of(s_start[b] + n - 1) - part_of(s_start[b]) + 1 : n;
        chunk_off[b] = nch;
    }
    __threadfence_block();
    __syncthreads();
    {
        const int per = ceil_div_i(B, kPlanThreads);
        const int lo = min(B, tid * per), hi = min(B, lo + per);
        int s = 0;
        for (int i = lo; i < hi; i++) s += chunk_off[i];
        s_scratch[tid] = s;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            int x = tid >= off ? s_scratch[tid - off] : 0;
            __syncthreads();
            s_scratch[tid] += x;
            __syncthreads();
        }
        int run = s_scratch[tid] - s;
        for (int i = lo; i < hi; i++) {
            int x = chunk_off[i];
            chunk_off[i] = run;
            run += x;
        }
        if (tid == 0) chunk_off[B] = s_scratch[kPlanThreads - 1];
    }
    __threadfence_block();
    __syncthreads();

    // items of each part, in request order
    for (int p = tid; p < num_parts; p += kPlanThreads) {
        const int e0 = edge(p), e1 = edge(p + 1);
        if (e1 <= e0) continue;
        int k = part_begin[p];
        const int bf = req_of(e0), bl = req_of(e1 - 1);
        for (int b = bf; b <= bl; b++) {
            const int S = s_start[b], n = s_start[b + 1] - S;
            if (n == 0) continue;
            const int f = sp.first(seq_lens[b]);
            const int lo = f + max(e0, S) - S, hi = f + min(e1, S + n) - S;
            const int L = sp.len(seq_lens[b]);
            const int nch = chunk_off[b + 1] - chunk_off[b];
            items[4 * k + 0] = b;
            items[4 * k + 1] = lo * kTileTokens;
            items[4 * k + 2] = min(hi * kTileTokens, L);
            items[4 * k + 3] = nch == 1 ? 1 : 0;
            k++;
        }
    }
    if (tid == 0) {
        plan[0] = kPlanMagic; plan[1] = 1; plan[2] = B; plan[3] = num_parts;
        plan[4] = part_begin[num_parts]; plan[5] = kTileTokens; plan[6] = max_items; plan[7] = 0;
    }
}

}  // namespace

hipError_t launch_plan(const int32_t *seq_lens, int32_t *plan, const PlanLayout &L,
                       const pa_decode_desc *d, hipStream_t stream)
{
    Span sp;
    sp.q_len = d->q_len;
    sp.window = d->window;
    sp.topk = d->topk;
    hipLaunchKernelGGL(pa_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, plan,
                       L.B, L.num_parts, L.max_items, d->num_splits, L.part_begin_off,
                       L.chunk_off_off, L.items_off, L.counters_off, L.n_counters, sp);
    return hipGetLastError();
}

}  // namespace pa
