// Split-KV MQA decode over the MLA 656-byte FP8 latent cache (D_qk = 576, D_v = 512,
// one KV head shared by G query heads, G a multiple of 16 up to 128), gfx950.
//
// Token layout (FlashMLA walk-through, section 数据加载, byte-layout table): 512 e4m3
// codes, 4 fp32 scales (one per 128 codes), 64 bf16 rope values.  The key is the 576
// dequantised values, the value is their first 512 (V shares the latent with K).
//
// One workgroup (4 waves, one per SIMD) = one (part, group of 64 query rows); it walks
// the part's items.  Query rows are (draft token qi, head g) pairs, row qi * G + g, so with
// several query tokens per request (a linear speculative draft) each wave's 16 rows share
// one draft token and its causal limit L - q_len + qi + 1.  The two head groups of a part run as workgroups 8 ids apart, i.e.
// on the same XCD at about the same time, so the second read of each KV tile is an L2
// hit (the FlashMLA walk-through shares one KV tile between two 64-head CTAs through a
// cluster, section 计算环节一; here the L2 of the XCD plays that role).  Per 32-token tile:
//   * raw tile: the 32 tokens' 656 bytes go HBM -> LDS by direct-to-LDS loads into a
//     3-slot ring (two tiles in flight while one is computed); each wave loads and
//     later dequantises 8 of the tokens, so it only ever waits for its own loads;
//   * conversion once per tile (not per head): e4m3 -> bf16 is exact, so the codes go
//     to a double-buffered bf16 K tile in LDS unscaled, with the token's 4 fp32 tile
//     scales in the row padding, and the rope values copied (FlashMLA walk-through:
//     dequantise to bf16 and run bf16 MMA with fp32 accumulation; section 计算环节一
//     for why dequantisation is the hot spot).  The scales are applied in fp32 instead
//     of being rounded into the bf16 values: S = sum_t scale_t (q_t . k_t) + q_rope .
//     k_rope over the four 128-dim tiles t, and for the value dims of tile t the
//     probabilities are multiplied by scale_t before the PV product;
//   * each wave owns 16 query heads: S^T[16 tok x 16 heads] = K . Q^T with bf16 MFMA
//     16x16x32 (K from the LDS tile, Q^T resident in 72 registers), an online softmax
//     per head column, and O^T[512 x 16 heads] += V^T . P^T with the V^T operand read
//     back transposed (ds_read_b64_tr_b16) from the same tile; O^T lives in 128
//     accumulation registers (the register-budget problem the FlashMLA walk-through
//     describes in section 计算环节二).
// The running max is only moved when a tile's max exceeds it by more than 2^8, so the
// 128-register rescale is rare; probabilities stay below 2^8 and the result is the
// same up to rounding (the reference cancels in the final normalisation).
//
// Sparse decode (FlashMLA walk-through, section 调度: the decode call takes sparse
// indices): the items then cover index slots, and slot k of request b names the key
// position indices[b][k].  The address of a listed token takes two dependent lookups
// (index, then block table), so they run ahead of the KV loads as per-lane vector loads
// (lanes 0-7: the wave's 8 tokens): tile j+4's indices and tile j+3's page ids are loaded
// while tile j is computed, and tile j+2's 8 tokens are gathered by direct-to-LDS loads
// with per-lane 64-bit addresses (41 chunks per token, 6 instructions per wave).  All of
// them go through the same in-order load counter as the KV tile, so the wait for tile
// j+1 also completes the lookups.  A slot outside the item or the request loads a dummy
// token that the conversion zeroes, and a per-tile bit mask of the real tokens is
// applied in the softmax.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define PA_LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = kWaves * kHeadsPerWave;   // 64
constexpr int kDqk = 576, kDv = 512;
constexpr int kTokBytes = 656;
constexpr int kChunks = kTokBytes / 16;            // 41 16-byte chunks per token
constexpr int kT = 32;                             // tokens per tile
constexpr int kTokPerWave = kT / kWaves;           // 8 tokens loaded / dequantised per wave
constexpr int kWaveChunks = kTokPerWave * kChunks; // 328
constexpr int kDmaPerWave = (kWaveChunks + 63) / 64;   // 6 direct-to-LDS loads per wave
constexpr int kRawTile = kT * kTokBytes;           // 20992
constexpr int kRawSlots = 3;
constexpr int kKRow = kDqk * 2 + 16;               // bf16 K row stride (padded) = 1168
constexpr int kKTile = kT * kKRow;                 // 37376
constexpr int kKSteps = kDqk / 32;                 // 18 (k = 32 per MFMA)
constexpr int kDvBlocks = kDv / 16;                // 32
constexpr float kLazyMax = 8.0f;                   // log2 units

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool SPARSE>
struct MlaCfg {
    // loads per wave and tile (sparse: the KV gather plus one index and one page-id load)
    static constexpr int kDmaPerTile = SPARSE ? kDmaPerWave + 2 : kDmaPerWave;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Barrier for LDS handoffs only: this wave's LDS writes are complete, then all waves
// meet.  (A full __syncthreads would also drain the in-flight KV loads.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// byte address of a shared-memory location, as LDS instructions take it
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(PA_LDS const void *)p;
}

__device__ __forceinline__ bf16x4 lds_tr16(const uint8_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PA_LDS bf16x4 *)((PA_LDS uint8_t *)p));
}

// SPARSE: index-slot items.  MASKED: a per-wave key range narrower than the item (draft
// tokens' causal limits, a sliding window); a separate instantiation, because the plain
// kernel sits at the register-file limit and any extra live value spills.
template <bool SPARSE, bool MASKED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void pa_mla_kernel(
    DecodeArgs a, const int32_t *__restrict__ plan, const int32_t *__restrict__ bt, int ngroups,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ indices)
{
    constexpr int kDmaPerTile = MlaCfg<SPARSE>::kDmaPerTile;
    __shared__ __attribute__((aligned(16))) uint8_t raw[kRawSlots][kRawTile];
    __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kKTile];
    __shared__ uint32_t s_valid[2];            // sparse: real-token bits of each K buffer
    // sparse lookups: [position | page id][tile % 4][wave][token]
    __shared__ int32_t s_look[SPARSE ? 2 * 4 * kWaves * kTokPerWave : 1];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    // workgroup id -> (part, head group): the head groups of one part are 8 ids apart
    const int wg = blockIdx.x;
    const int part = (wg / (8 * ngroups)) * 8 + wg % 8;
    const int group = (wg / 8) % ngroups;
    if (part >= a.num_parts) return;               // padding of the last id block
    const int G = a.G, Hq = a.Hkv * a.G, nq = a.q_len;
    const int row0 = group * kHeadsPerWG + wave * kHeadsPerWave;   // first query row
    const bool active = row0 < G * nq;             // wave-uniform
    const int qi = row0 / G;                       // the wave's draft token (G % 16 == 0)
    const int head0 = row0 - qi * G;               // its first head
    const int col = lane & 15, g4 = lane >> 4;     // MFMA column (head), lane group

    // lane byte offset of chunk x = 64 i + lane (token x / 41, chunk x % 41) inside the
    // 8 token rows a wave loads per tile (the sparse gather recomputes its split)
    int dma_off[kDmaPerWave];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; i++) {
        const int x = 64 * i + lane;
        const int tt = x / kChunks, c = x - tt * kChunks;
        dma_off[i] = SPARSE ? 0 : tt * (int)a.s_tok_b + 16 * c;
    }

    const int ib = plan[a.part_begin_off + part];
    const int ie = plan[a.part_begin_off + part + 1];

    for (int it = ib; it < ie; it++) {
        const int b = plan[a.items_off + 4 * it + 0];
        const int t0 = plan[a.items_off + 4 * it + 1];
        const int t1 = plan[a.items_off + 4 * it + 2];
        const int flags = plan[a.items_off + 4 * it + 3];
        const int ntiles = (t1 - t0 + kT - 1) / kT;
        // causal limit of the wave's draft token and the first key its window leaves
        int tlim = t1, tlo = 0;
        if (MASKED) {
            const int L = seq_lens[b];
            if (nq > 1) tlim = min(t1, L - (nq - 1 - qi));
            if (a.window > 0) tlo = max(0, L - nq + qi - a.window + 1);
        }

        // sparse lookups, lane l: token l % 8 of the wave's 8 in tile j, index slot k.  They
        // go to shared memory by direct-to-LDS loads (no registers live across the tile
        // compute; the loads complete in order with the KV gathers) and are read back by
        // inline asm (which the compiler does not make wait for the gathers in flight).
        const int Lb = SPARSE ? seq_lens[b] : 0;
        auto sp_slot = [&](int j) { return t0 + kT * j + kTokPerWave * wave + (lane & 7); };
        auto sp_ok = [&](int j, int pos) { return sp_slot(j) < t1 && pos >= 0 && pos < Lb; };
        auto look = [&](int which, int j) { return &s_look[((which * 4 + (j & 3)) * kWaves + wave) * kTokPerWave]; };
        auto sp_issue_pos = [&](int j) {           // slots past the row: its last entry
            if (lane < kTokPerWave)
                __builtin_amdgcn_global_load_lds((const void *)(indices + (int64_t)b * a.topk + min(sp_slot(j), a.topk - 1)),
                                                 (PA_LDS void *)look(0, j), 4, 0, 0);
        };
        auto sp_issue_page = [&](int j, int pos) { // no real token: the row's first page
            if (lane < kTokPerWave)
                __builtin_amdgcn_global_load_lds(
                    (const void *)(bt + (int64_t)b * a.max_pages + (sp_ok(j, pos) ? pos >> a.page_shift : 0)),
                    (PA_LDS void *)look(1, j), 4, 0, 0);
        };
        auto sp_read = [&](int which, int j) {     // issue only: complete after lgkm_wait
            int v;
            asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(lds_addr(look(which, j)) + 4 * (lane & 7)));
            return v;
        };
        auto lgkm_wait = [](int &x, int &y, int &z) {
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x), "+v"(y), "+v"(z)::"memory");
        };

        // ---- direct-to-LDS load of this wave's 8 tokens of tile j into raw slot s (buffer
        //      loads over the 8 token rows: one 32-bit lane offset per instruction)
        // sparse: gather of the wave's 8 listed tokens of tile j (position pos and page id
        // page in lane l % 8) into raw slot s; returns the bits of the real tokens.  A
        // token that is not real loads the first token of page 0 instead.
        auto dma_sparse = [&](int j, int s, int pos, int page) {
            const bool ok = sp_ok(j, pos);
            const int64_t off = ok ? (int64_t)page * a.s_page_b +
                                         (int64_t)(pos & ((1 << a.page_shift) - 1)) * a.s_tok_b
                                   : 0;
            const int lo = (int)(uint32_t)off, hi = (int)(off >> 32);
            uint8_t *dst = &raw[s][wave * kWaveChunks * 16];
#pragma unroll
            for (int i = 0; i < kDmaPerWave; i++) {
                // chunk x = 64 i + lane: token x / 41 (as x * 1599 >> 16, exact for x < 1681)
                const int x = 64 * i + lane;
                const int tt = (x * 1599) >> 16, c = x - kChunks * tt;
                const uint32_t tlo = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * tt, lo);
                const uint32_t thi = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * tt, hi);
                const uint8_t *g = a.k_pool + (int64_t)(((uint64_t)thi << 32) | tlo) + 16 * c;
                if (64 * i + lane < kWaveChunks)
                    __builtin_amdgcn_global_load_lds((const void *)g, (PA_LDS void *)(dst + 64 * 16 * i), 16,
                                                     0, 0);
            }
            return (uint32_t)__ballot(ok) & 0xFFu;
        };

        auto dma_tile = [&](int j, int s) {
            const int jc = j < ntiles ? j : ntiles - 1;     // past the end: reload the last tile
            int tw = t0 + kT * jc + kTokPerWave * wave;     // first of the wave's 8 tokens
            if (tw >= t1) tw = (t1 - 1) & ~(kTokPerWave - 1);
            const int page = bt[(int64_t)b * a.max_pages + (tw >> a.page_shift)];
            const int slot0 = tw & ((1 << a.page_shift) - 1);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.k_pool + (int64_t)page * a.s_page_b + (int64_t)slot0 * a.s_tok_b), (short)0,
                kTokPerWave * (int)a.s_tok_b, 0x00020000);
            uint8_t *dst = &raw[s][wave * kWaveChunks * 16];
#pragma unroll
            for (int i = 0; i < kDmaPerWave; i++) {
                if (64 * i + lane < kWaveChunks)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (PA_LDS void *)(dst + 64 * 16 * i), 16,
                                                             dma_off[i], 0, 0, 0);
            }
        };

        // ---- convert this wave's 8 tokens of raw slot s into K tile buffer kb.  Lane l
        //      converts latent dims 8l..8l+7 of one token per round (8-byte reads, 16-byte
        //      writes: 16 neighbouring lanes touch 256 contiguous bytes, no bank conflicts);
        //      then the rope chunks (lane: token l / 8, chunk l % 8) and the 4 tile scales
        //      (lanes 0-7, into the row padding).  Rows of tokens >= t1 become 0.
        //      Sparse: vm holds the bits of the wave's real tokens (byte `wave` of the
        //      tile's mask); the other rows become 0.
        auto dequant_tile = [&](int j, int s, int kb, uint32_t vm) {
            const int row0 = kTokPerWave * wave;
            const int tbase = t0 + kT * j + row0;
            auto dead = [&](int tt) { return SPARSE ? ((vm >> tt) & 1u) == 0 : tbase + tt >= t1; };
            if (SPARSE && lane == 0) ((uint8_t *)&s_valid[kb])[wave] = (uint8_t)vm;
            // the raw slot is read by inline asm: the compiler cannot tell these reads from
            // the direct-to-LDS writes of later tiles still in flight, and before plain
            // reads it would wait for those too (all loads of this wave), emptying the ring
            const uint32_t rbase = lds_addr(&raw[s][row0 * kTokBytes]);
            uint64_t w[kTokPerWave];
            u32x4 rope, scl;
#pragma unroll
            for (int tt = 0; tt < kTokPerWave; tt++)
                asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(w[tt]) : "v"(rbase + 8 * lane), "n"(tt * kTokBytes));
            asm volatile("ds_read_b128 %0, %1 offset:528" : "=v"(rope)
                         : "v"(rbase + (lane >> 3) * kTokBytes + 16 * (lane & 7)));
            asm volatile("ds_read_b128 %0, %1 offset:512" : "=v"(scl) : "v"(rbase + (lane & 7) * kTokBytes));
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]),
                           "+v"(w[6]), "+v"(w[7]), "+v"(rope), "+v"(scl)::"memory");
#pragma unroll
            for (int tt = 0; tt < kTokPerWave; tt++) {
                const int lo = (int)(uint32_t)w[tt], hi = (int)(w[tt] >> 32);
                bf16x8 o;
                const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
                const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
                const bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
                const bf16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
                o[0] = b0[0]; o[1] = b0[1]; o[2] = b1[0]; o[3] = b1[1];
                o[4] = b2[0]; o[5] = b2[1]; o[6] = b3[0]; o[7] = b3[1];
                if (dead(tt)) o = bf16x8{};
                *(bf16x8 *)(&ktile[kb][(row0 + tt) * kKRow + 16 * lane]) = o;
            }
            {
                const int tt = lane >> 3, c = lane & 7;
                if (dead(tt)) rope = u32x4{0, 0, 0, 0};
                *(u32x4 *)(&ktile[kb][(row0 + tt) * kKRow + (512 + 8 * c) * 2]) = rope;
            }
            if (lane < kTokPerWave) {
                if (dead(lane)) scl = u32x4{0, 0, 0, 0};
                *(u32x4 *)(&ktile[kb][(row0 + lane) * kKRow + kDqk * 2]) = scl;
            }
        };

        // ---- Q^T operand of this wave's 32 heads (B of the 32x32x16 MFMA), resident
        bf16x8 qop[kKSteps];
        if (active) {
            const uint16_t *qrow = a.q + (((int64_t)b * nq + qi) * Hq + head0 + col) * kDqk;
#pragma unroll
            for (int s = 0; s < kKSteps; s++) qop[s] = *(const bf16x8 *)(qrow + 32 * s + 8 * g4);
        }

        f32x4 acc[kDvBlocks];
#pragma unroll
        for (int i = 0; i < kDvBlocks; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY;     // reference max (log2 domain) of head `col`
        float l = 0.f;

        if (ntiles > 0) {
            // sparse pipeline at the top of tile j: the positions of tiles j+2 and j+3 and
            // the page ids of tile j+2 are in shared memory, vm1 = real-token bits of j+1
            uint32_t vm0 = 0, vm1 = 0, vm2 = 0;
            if (SPARSE) {
                // positions of tiles 0-3, page ids of tiles 0-2, gathers of tiles 0 and 1
                for (int t = 0; t < 4; t++) sp_issue_pos(t);
                wait_vmcnt<0>();
                int p0 = sp_read(0, 0), p1 = sp_read(0, 1), p2 = sp_read(0, 2);
                lgkm_wait(p0, p1, p2);
                sp_issue_page(0, p0);
                sp_issue_page(1, p1);
                sp_issue_page(2, p2);
                wait_vmcnt<0>();
                int g0 = sp_read(1, 0), g1 = sp_read(1, 1), unused = 0;
                lgkm_wait(g0, g1, unused);
                vm0 = dma_sparse(0, 0, p0, g0);
                vm1 = dma_sparse(1, 1, p1, g1);
                wait_vmcnt<kDmaPerWave>();        // tile 0 done (tile 1's gather is younger)
            } else {
                dma_tile(0, 0);
                dma_tile(1, 1);
                wait_vmcnt<kDmaPerTile>();        // own loads of tile 0 done
            }
            dequant_tile(0, 0, 0, vm0);
            lds_barrier();

            // The tile loop never rescales O^T itself: when a tile's max exceeds the
            // reference by more than 2^8 it leaves (before that tile's PV), the rescale
            // runs outside, and the loop resumes at the same tile.  Inside the loop O^T is
            // only touched by MFMAs, so it stays in the accumulation registers.
            int j = 0;
            int dma_next = 2;                     // next tile whose loads are not issued yet
            float bm_exit = -INFINITY;
            for (;;) {
            for (; j < ntiles; j++) {
                // tile j+2's loads go out before the compute of tile j (once per tile, also
                // when the loop resumes at j after a rescale)
                if (dma_next == j + 2) {
                    if (SPARSE) {
                        // the previous tile's lookups are done (tile j+1's gather is
                        // younger); issue tile j+3's page ids and tile j+4's positions
                        // (the next tile waits for these, not for this tile's KV), then
                        // the gather of tile j+2
                        wait_vmcnt<kDmaPerWave>();
                        int p3 = sp_read(0, j + 3), p2 = sp_read(0, j + 2), g2 = sp_read(1, j + 2);
                        lgkm_wait(p3, p2, g2);
                        sp_issue_page(j + 3, p3);
                        sp_issue_pos(j + 4);
                        vm2 = dma_sparse(j + 2, (j + 2) % kRawSlots, p2, g2);
                    } else {
                        dma_tile(j + 2, (j + 2) % kRawSlots);
                    }
                    dma_next++;
                }
                const uint8_t *kt = ktile[j & 1];

                if (active) {
                    // ---- S^T = K . Q^T for the two 16-token row blocks (rows 16sb + 4g4 + r):
                    //      one partial per 128-dim scale tile (k-steps 4t..4t+3) and one for
                    //      the rope dims (k-steps 16, 17), combined with the tile scales in fp32
                    // Per 16-token row block: 18 MFMA steps whose K operand is read from LDS
                    // two steps ahead; the scheduling barriers pin that order (one wave per
                    // SIMD: nothing else hides the LDS latency).
                    f32x4 st[2];
                    f32x4 sc4[2][4];       // scales of this lane's 8 tokens: [sb][r] -> 4 tiles
#pragma unroll
                    for (int sb = 0; sb < 2; sb++) {
                        f32x4 part[5];
#pragma unroll
                        for (int t = 0; t < 5; t++) part[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                        const uint8_t *kbase = kt + (16 * sb + col) * kKRow + 16 * g4;
                        bf16x8 kf[3];
                        kf[0] = *(const bf16x8 *)kbase;
                        kf[1] = *(const bf16x8 *)(kbase + 64);
#pragma unroll
                        for (int ks = 0; ks < kKSteps; ks++) {
                            if (ks + 2 < kKSteps) kf[(ks + 2) % 3] = *(const bf16x8 *)(kbase + 64 * (ks + 2));
                            const int t = ks < 16 ? ks / 4 : 4;
                            part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % 3], qop[ks], part[t], 0, 0, 0);
                            __builtin_amdgcn_sched_barrier(0);
                        }
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            sc4[sb][r] = *(const f32x4 *)(kt + (16 * sb + 4 * g4 + r) * kKRow + kDqk * 2);
                            float x = part[4][r];
#pragma unroll
                            for (int t = 0; t < 4; t++) x += sc4[sb][r][t] * part[t][r];
                            st[sb][r] = x;
                        }
                    }
                    // ---- online softmax with a lazily moved reference
                    float bm = -INFINITY;
                    float sv[8];
                    const uint32_t vmask = SPARSE ? s_valid[j & 1] : 0u;
#pragma unroll
                    for (int r = 0; r < 8; r++) {
                        const int row = 16 * (r >> 2) + 4 * g4 + (r & 3);
                        const int tok = t0 + kT * j + row;
                        const bool vis = SPARSE ? ((vmask >> row) & 1u) != 0
                                                : MASKED ? (tok < tlim && tok >= tlo) : tok < t1;
                        sv[r] = vis ? st[r >> 2][r & 3] * a.scale_log2 : -INFINITY;
                        bm = fmaxf(bm, sv[r]);
                    }
                    bm = fmaxf(bm, __shfl_xor(bm, 16));
                    bm = fmaxf(bm, __shfl_xor(bm, 32));
                    if (__any(bm > m + kLazyMax)) {
                        bm_exit = bm;
                        break;
                    }
                    const float mref = m == -INFINITY ? 0.f : m;
                    bf16x8 pbt[4];         // P times the scale of value tile t, per token
                    float ps = 0.f;
#pragma unroll
                    for (int r = 0; r < 8; r++) {
                        const float pr = fast_exp2(sv[r] - mref);
                        ps += pr;
#pragma unroll
                        for (int t = 0; t < 4; t++) pbt[t][r] = (__bf16)(pr * sc4[r >> 2][r & 3][t]);
                    }
                    l += ps;
                    // ---- O^T += V^T . P^T; k = 8g4 + r <-> token (r < 4 ? 4g4 + r : 16 + 4g4 + r - 4)
                    const uint8_t *vbase = kt + (4 * g4 + (col >> 2)) * kKRow + 4 * (col & 3) * 2;
                    auto read_vt = [&](int db) {
                        const bf16x4 lo = lds_tr16(vbase + 32 * db);
                        const bf16x4 hi = lds_tr16(vbase + 16 * kKRow + 32 * db);
                        bf16x8 va;
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            va[e] = lo[e];
                            va[4 + e] = hi[e];
                        }
                        return va;
                    };
                    bf16x8 vf[3];
                    vf[0] = read_vt(0);
                    vf[1] = read_vt(1);
#pragma unroll
                    for (int db = 0; db < kDvBlocks; db++) {
                        if (db + 2 < kDvBlocks) vf[(db + 2) % 3] = read_vt(db + 2);
                        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db % 3], pbt[db >> 3], acc[db], 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // ---- next tile: own loads of tile j+1 done (tile j+2's are younger), then
                //      dequantise it into the other K buffer
                wait_vmcnt<kDmaPerTile>();
                dequant_tile(j + 1, (j + 1) % kRawSlots, (j + 1) & 1, vm1);
                vm1 = vm2;
                lds_barrier();
            }
            if (j >= ntiles) break;
            // move the reference to this tile's max and rescale (rare); tile j is redone
            {
                const float mn = fmaxf(m, bm_exit);
                const float alpha = fast_exp2(m - mn);   // m = -inf: 0
                m = mn;
                l *= alpha;
#pragma unroll
                for (int i = 0; i < kDvBlocks; i++) acc[i] *= alpha;
            }
            }
            wait_vmcnt<0>();
        }

        // ---- epilogue: this wave's heads are complete for this item
        if (active) {
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            const int head = head0 + col;
            float inv, lse_v;
            const float sk = (a.sinks && (flags & 1)) ? a.sinks[head] * 1.4426950408889634f : -INFINITY;
            const float M2 = fmaxf(m, sk);
            if (M2 == -INFINITY || (sk == -INFINITY && l == 0.f)) {
                inv = 0.f;                                   // nothing to attend to
                lse_v = -INFINITY;
            } else {
                // a sink (whole-request items only; split requests get it in the merge)
                // joins the denominator: den = l 2^(m - M2) + 2^(sk - M2)
                const float fm = fast_exp2(m - M2);          // m = -inf: 0
                const float den = l * fm + fast_exp2(sk - M2);
                inv = fm / den;
                lse_v = (M2 + log2f(den)) * 0.69314718055994530942f;
            }
            const int64_t qr = (int64_t)qi * Hq + head;      // query row within the request
            const int64_t row = (int64_t)b * nq * Hq + qr;
            // O^T layout: lane holds dims 16db + 4g4 + e of head `col`
            if (flags & 1) {
                uint16_t *orow = a.out + row * kDv + 4 * g4;
#pragma unroll
                for (int db = 0; db < kDvBlocks; db++) {
                    bf16x4 o;
#pragma unroll
                    for (int e = 0; e < 4; e++) o[e] = (__bf16)(acc[db][e] * inv);
                    *(bf16x4 *)(orow + 16 * db) = o;
                }
                if (g4 == 0) a.lse[row] = lse_v;
            } else {
                const int64_t prow = (int64_t)it * nq * Hq + qr;
                float *orow = a.ws_o + prow * kDv + 4 * g4;
#pragma unroll
                for (int db = 0; db < kDvBlocks; db++) *(f32x4 *)(orow + 16 * db) = acc[db] * inv;
                if (g4 == 0) a.ws_lse[prow] = lse_v;
            }
        }
        lds_barrier();
    }
}

}  // namespace

hipError_t launch_mla(const DecodeArgs &a, hipStream_t stream)
{
    const int ngroups = (a.G * a.q_len + kHeadsPerWG - 1) / kHeadsPerWG;
    const int nwg = (a.num_parts + 7) / 8 * 8 * ngroups;
    if (a.topk > 0)
        hipLaunchKernelGGL((pa_mla_kernel<true, false>), dim3(nwg), dim3(kThreads), 0, stream, a,
                           a.plan, a.block_table, ngroups, a.seq_lens, a.indices);
    else if (a.q_len > 1 || a.window > 0)
        hipLaunchKernelGGL((pa_mla_kernel<false, true>), dim3(nwg), dim3(kThreads), 0, stream, a,
                           a.plan, a.block_table, ngroups, a.seq_lens, a.indices);
    else
        hipLaunchKernelGGL((pa_mla_kernel<false, false>), dim3(nwg), dim3(kThreads), 0, stream, a,
                           a.plan, a.block_table, ngroups, a.seq_lens, a.indices);
    return hipGetLastError();
}

}  // namespace pa
