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

constexpr int kPlanThreads = 512;

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

constexpr int kPlanWaves = kPlanThreads / 64;

// inclusive scan of x across the 64 lanes of a wave: DPP row shifts by 1, 2, 4, 8 inside
// each row of 16 lanes, then the row broadcasts of lanes 15 and 31 (lanes a shift or
// broadcast does not reach add 0)
__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return x;
}

// Exclusive scan of v[0..n) in LDS, in place; v[n] = the total, which is also returned.
// Each thread sums a run of ceil(n / kPlanThreads) elements, the runs are scanned within
// each wave and across the waves (by one wave): two barriers.  All threads call.
__device__ int block_exclusive_scan(int *v, int n, int *wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (n + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int s = 0;
    for (int i = lo; i < hi; i++) s += v[i];
    const int incl = wave_inclusive_scan(s);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (w == 0) {
        const int x = lane < kPlanWaves ? wsum[lane] : 0;
        const int y = wave_inclusive_scan(x);
        if (lane < kPlanWaves) wsum[kPlanWaves + lane] = y - x;       // exclusive wave offsets
        if (lane == kPlanWaves - 1) wsum[2 * kPlanWaves] = y;          // total
    }
    __syncthreads();
    int run = wsum[kPlanWaves + w] + incl - s;
    for (int i = lo; i < hi; i++) {
        const int x = v[i];
        v[i] = run;
        run += x;
    }
    const int total = wsum[2 * kPlanWaves];
    if (tid == 0) v[n] = total;
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(kPlanThreads) void pa_plan_kernel(
    const int32_t *__restrict__ seq_lens, int32_t *__restrict__ plan, int B, int num_parts,
    int max_items, int num_splits, int part_begin_off, int chunk_off_off, int items_off,
    int counters_off, int n_counters, Span sp)
{
    __shared__ int s_start[kMaxBatch + 1];   // tile prefix S_b
    __shared__ int s_chunk[kMaxBatch + 1];   // chunk prefix (chunk_off)
    __shared__ int s_part[kMaxPlanParts + 1];   // item prefix per part (part_begin)
    __shared__ int s_len[kMaxBatch];         // seq_lens
    __shared__ int s_wsum[2 * kPlanWaves + 1];
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

    // ---- balanced parts: tile counts and their prefix (everything stays in LDS)
    for (int b = tid; b < B; b += kPlanThreads) {
        const int L = seq_lens[b];
        s_len[b] = L;
        s_start[b] = sp.tiles(L);
    }
    for (int p = tid; p <= num_parts; p += kPlanThreads) s_part[p] = 0;
    __syncthreads();
    const int N = block_exclusive_scan(s_start, B, s_wsum);

    // Part p owns global tiles [edge(p), edge(p + 1)), edge(p) = floor(p N / P); the part
    // holding tile x (0 <= x < N) is the largest p with edge(p) <= x, floor(((x + 1) P - 1) / N).
    // Both in double: the numerators stay below 2^53 and the quotients' fractional parts are
    // multiples of 1 / P or 1 / N, far above the rounding error, so the floors are exact.
    const int P = num_parts;
    auto edge = [&](int p) -> int { return (int)(((double)p * (double)N) / (double)P); };
    auto part_of = [&](int x) -> int { return (int)(((double)(x + 1) * (double)P - 1.0) / (double)N); };
    // When N >= P every part holds at least one tile, so the parts a request touches are
    // consecutive and all non-empty: one chunk per part.  Otherwise every non-empty part
    // holds exactly one tile and a request has one chunk per tile.
    const bool wide = N >= P;

    // chunks per request; each chunk counts one item of its part
    for (int b = tid; b < B; b += kPlanThreads) {
        const int S = s_start[b], n = s_start[b + 1] - S;
        int nch = 0;
        if (n > 0) {
            const int pf = part_of(S);
            nch = wide ? part_of(S + n - 1) - pf + 1 : n;
            for (int j = 0; j < nch; j++) atomicAdd(&s_part[wide ? pf + j : part_of(S + j)], 1);
        }
        s_chunk[b] = nch;
    }
    __syncthreads();
    const int n_items = block_exclusive_scan(s_part, P, s_wsum);
    block_exclusive_scan(s_chunk, B, s_wsum);
    for (int p = tid; p <= P; p += kPlanThreads) part_begin[p] = s_part[p];
    for (int b = tid; b <= B; b += kPlanThreads) chunk_off[b] = s_chunk[b];

    // items: items are numbered in (request, part) order along the tile axis, so chunk j of
    // request b is item chunk_off[b] + j
    for (int b = tid; b < B; b += kPlanThreads) {
        const int S = s_start[b], n = s_start[b + 1] - S;
        if (n == 0) continue;
        const int L = s_len[b];
        const int f = sp.first(L), Lk = sp.len(L);
        const int c0 = s_chunk[b], nch = s_chunk[b + 1] - c0;
        const int pf = wide ? part_of(S) : 0;
        for (int j = 0; j < nch; j++) {
            int lo, hi;                                  // global tiles of the chunk
            if (wide) {
                lo = max(edge(pf + j), S);
                hi = min(edge(pf + j + 1), S + n);
            } else {
                lo = S + j;
                hi = lo + 1;
            }
            int32_t *it = items + 4 * (c0 + j);
            it[0] = b;
            it[1] = (f + lo - S) * kTileTokens;
            it[2] = min((f + hi - S) * kTileTokens, Lk);
            it[3] = nch == 1 ? 1 : 0;
        }
    }
    if (tid == 0) {
        plan[0] = kPlanMagic; plan[1] = 1; plan[2] = B; plan[3] = P;
        plan[4] = n_items; plan[5] = kTileTokens; plan[6] = max_items; plan[7] = 0;
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
