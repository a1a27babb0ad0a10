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
// one draft token and its causal limit L - q_len + qi + 1.  The two head groups of a part
// run as workgroups 8 ids apart, i.e. on the same XCD at about the same time, so the
// second read of each KV tile is an L2 hit (the FlashMLA walk-through shares one KV tile
// between two 64-head CTAs through a cluster, section 计算环节一; here the L2 of the XCD
// plays that role).
//
// Per 32-token tile:
//   * the tokens' 656 bytes go HBM -> LDS by direct-to-LDS loads (one instruction per
//     token, 41 lanes of 16 bytes; a token that is not real reads as zeros) into a 6-slot
//     ring of 672-byte rows, so each tile's loads are issued 5 tiles ahead;
//   * the FP8 codes stay FP8 in LDS: each wave converts the MFMA operands it reads to
//     bf16 in registers right before the MFMA (e4m3 -> bf16 is exact).  A bf16 copy of
//     the tile would cost twice the LDS reads plus its writes, and LDS bandwidth, not the
//     matrix cores, bounds this loop on gfx950.  (The FlashMLA walk-through dequantises
//     to bf16 and runs bf16 MMA with fp32 accumulation, section 计算环节一.)  The scales
//     are applied in fp32 instead of being rounded into the bf16 values:
//     S = sum_t scale_t (q_t . k_t) + q_rope . k_rope over the four 128-dim tiles t, and
//     for the value dims of tile t the probabilities are multiplied by scale_t before PV;
//   * each wave owns 16 query heads: S^T[32 tok x 16 heads] = K . Q^T with bf16 MFMA
//     16x16x32 (Q^T resident), an online softmax per head column, and
//     O^T[512 x 16 heads] += V^T . P^T with V^T read transposed from the FP8 codes
//     (ds_read_b64_tr_b8); O^T lives in 128 accumulation registers (the register-budget
//     problem the FlashMLA walk-through describes in section 计算环节二).
// Operand layouts.  QK row block sb (0, 1) of the A operand holds, in MFMA row m = 4g + r,
// token 8g + 4sb + r, so lane group g of the S^T result holds tokens 8g..8g+7: exactly the
// k slots the same lanes feed to the PV MFMA (B = P^T, k = 8g + j), and the transposed
// read returns tokens 8g..8g+7 of one value dim per lane.  A 16-byte read of the codes
// feeds two k-steps (dims 64p + 16g + 0..7 and + 8..15), and Q^T is loaded in the same
// order.
// With one wave per SIMD nothing else hides a wave's VALU and LDS work behind its
// MFMAs, so the tile loop is software-pipelined by hand (the FlashMLA walk-through
// overlaps the softmax of one tile with the matrix products of another across two
// warpgroups, section 计算环节二; here one wave interleaves the two streams):
//   top of tile j: the loads of tile j+1 are in; workgroup barrier; loads of tile j+5 out;
//   phase 1: the QK MFMAs of tile j+1, with the softmax of tile j between them;
//   phase 2: the PV MFMAs of tile j.
// The running max is only moved when a tile's max exceeds it by more than 2^8, so the
// 128-register rescale is rare; probabilities stay below 2^8 and the result is the
// same up to rounding (the reference cancels in the final normalisation).
//
// Sparse decode (FlashMLA walk-through, section 调度: the decode call takes sparse
// indices): the items then cover index slots, and slot k of request b names the key
// position indices[b][k].  The address of a listed token takes two dependent lookups
// (index, then block table); lanes 0-7 of each wave (its 8 tokens of a tile) load them
// direct to LDS, positions 8 tiles and page ids 4 tiles ahead of the tile's own loads,
// so that every wait for them is one the KV ring does anyway.  A slot outside the item or
// the request loads nothing (zeros), and a per-tile bit mask of the real tokens is
// applied in the softmax.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define PA_LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = kWaves * kHeadsPerWave;   // 64
constexpr int kDqk = 576, kDv = 512;
constexpr int kTokBytes = 656;
constexpr int kChunks = kTokBytes / 16;            // 41 16-byte chunks per token
constexpr int kT = 32;                             // tokens per tile
constexpr int kTokPerWave = kT / kWaves;           // 8 tokens loaded per wave and tile
constexpr int kRawRow = 672;                       // LDS row of a token (656 + 16)
constexpr int kRawTile = kT * kRawRow;             // 21504
constexpr int kRawSlots = 6;                       // tile ring
constexpr int kAhead = kRawSlots - 2;              // lookups: page ids 4, positions 8 tiles ahead
constexpr int kLookRing = 16;                      // lookup slots (tiles) per wave
constexpr int kDvBlocks = kDv / 16;                // 32 PV MFMAs per tile and wave
constexpr float kLazyMax = 8.0f;                   // log2 units

static_assert(kRawSlots >= 4, "the tile loop keeps tiles j, j+1 and loads in flight");
static_assert(kLookRing > 2 * kAhead, "lookup ring");

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool SPARSE>
struct MlaCfg {
    // loads per wave and tile: one per token (sparse: plus one page-id and one index load)
    static constexpr int kLoadsPerTile = SPARSE ? kTokPerWave + 2 : kTokPerWave;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Barrier for LDS handoffs only: this wave's LDS accesses are complete, then all waves
// meet.  (A full __syncthreads would also drain the in-flight KV loads.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// byte address of a shared-memory location, as LDS instructions take it
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(PA_LDS const void *)p;
}

// Direct-to-LDS loads, issued as inline asm (M0 = the LDS address of lane 0's data; lane
// i's goes i * size bytes further).  The compiler then does not see them as LDS writes:
// it neither makes unrelated LDS accesses wait for them (its alias tracking of such
// loads gives up across loop iterations and waits for all of them) nor counts them;
// every wait for them in this file is explicit.  Nothing else here uses M0.
__device__ __forceinline__ void lds_dma_buf16(__amdgpu_buffer_rsrc_t rs, int voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma_glb4(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}

// 8 e4m3 codes (two words) -> 8 bf16 (exact)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi)
{
    const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 o;
    o[0] = b0[0]; o[1] = b0[1]; o[2] = b1[0]; o[3] = b1[1];
    o[4] = b2[0]; o[5] = b2[1]; o[6] = b3[0]; o[7] = b3[1];
    return o;
}

// max / sum over the lanes l, l^16, l^32, l^48 (the 4 row groups of one MFMA column),
// through the row-swap permutes (no LDS); the result is the same in all four lanes
__device__ __forceinline__ float col_max(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float col_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Q as two fp8 terms for the scaled fp8 MFMA: hi = e4m3(v 2^-e_hi), lo = e4m3((v - hi
// 2^e_hi) 2^-e_lo), with e the power of two that brings the max |.| over the head's 128
// dims (this lane's 32 and those of lanes l^16, l^32, l^48) into [128, 256), within the
// E8M0 range.  A bf16 value has 8 significant bits and each term keeps 4, so hi + lo is v
// exactly for every v within 2^13 of the maximum, and within 2^-21 of it otherwise.
__device__ __forceinline__ int split_exp(float mx)
{
    return max(__builtin_amdgcn_frexp_expf(col_max(mx)) - 8, -127);
}
__device__ __forceinline__ int fp8x4_code(const float *v, int e)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(v[0], -e), __builtin_amdgcn_ldexpf(v[1], -e), 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(v[2], -e), __builtin_amdgcn_ldexpf(v[3], -e), w, true);
}
__device__ __forceinline__ int q_split_exp(const float (&v)[32])
{
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i++) mx = fmaxf(mx, fabsf(v[i]));
    return split_exp(mx);
}
__device__ __forceinline__ int q_split_lo(const float (&v)[32], int e_hi, i32x8 &hi, i32x8 &lo)
{
    float r[32], mx = 0.f;
#pragma unroll
    for (int d = 0; d < 8; d++) {
        const int w = fp8x4_code(&v[4 * d], e_hi);
        hi[d] = w;
        const f32x2 x0 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const f32x2 x1 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        r[4 * d + 0] = v[4 * d + 0] - __builtin_amdgcn_ldexpf(x0[0], e_hi);
        r[4 * d + 1] = v[4 * d + 1] - __builtin_amdgcn_ldexpf(x0[1], e_hi);
        r[4 * d + 2] = v[4 * d + 2] - __builtin_amdgcn_ldexpf(x1[0], e_hi);
        r[4 * d + 3] = v[4 * d + 3] - __builtin_amdgcn_ldexpf(x1[1], e_hi);
    }
#pragma unroll
    for (int i = 0; i < 32; i++) mx = fmaxf(mx, fabsf(r[i]));
    const int e_lo = split_exp(mx);
#pragma unroll
    for (int d = 0; d < 8; d++) lo[d] = fp8x4_code(&r[4 * d], e_lo);
    return e_lo;
}

// scaled fp8 MFMA 16x16x128 (both operands e4m3): A unscaled, B scaled by byte u of sc
__device__ __forceinline__ f32x4 mfma_fp8_q(int u, const i32x8 &a, const i32x8 &b, const f32x4 &c, uint32_t sc)
{
    switch (u) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0x7F7F7F7F, 0, (int)sc);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0x7F7F7F7F, 1, (int)sc);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0x7F7F7F7F, 2, (int)sc);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0x7F7F7F7F, 3, (int)sc);
    }
}

// SPARSE: index-slot items.  MASKED: a per-wave key range narrower than the item (draft
// tokens' causal limits, a sliding window); a separate instantiation, because the plain
// kernel sits near the register-file limit.
template <bool SPARSE, bool MASKED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void pa_mla_kernel(
    DecodeArgs a, const int32_t *__restrict__ plan, const int32_t *__restrict__ bt, int ngroups,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ indices)
{
    constexpr int kLoadsPerTile = MlaCfg<SPARSE>::kLoadsPerTile;
    __shared__ __attribute__((aligned(16))) uint8_t raw[kRawSlots][kRawTile];
    __shared__ uint32_t s_valid[kRawSlots];    // sparse: real-token bits of each slot
    // sparse lookups: [position | page id][tile % 16][wave][token]
    __shared__ int32_t s_look[SPARSE ? 2 * kLookRing * kWaves * kTokPerWave : 1];

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
    const int page_mask = (1 << a.page_shift) - 1;

    // LDS byte offsets inside a tile slot: the QK operand rows of row block 0 (token
    // 8(col/4) + col%4, at this lane's 16 bytes of each 64-dim group; row block 1 is 4
    // rows further), the scale rows of this lane's tokens 8g4 + j, and the transposed PV
    // read (lane pair 2r, 2r+1 of a 16-lane block supplies row 8g4 + r, bytes 0-7 and
    // 8-15 of the block's 16 value dims)
    const uint32_t qk_off0 = (uint32_t)((8 * (col >> 2) + (col & 3)) * kRawRow + 16 * g4);
    const uint32_t sc_off = (uint32_t)(8 * g4 * kRawRow + 512);
    const uint32_t pv_off = (uint32_t)((8 * g4 + ((lane & 15) >> 1)) * kRawRow + 8 * (lane & 1));

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

        // ---- sparse lookups, lane l < 8: token l of the wave's 8 in tile j, index slot k
        const int Lb = SPARSE ? seq_lens[b] : 0;
        auto sp_slot = [&](int j) { return t0 + kT * j + kTokPerWave * wave + (lane & 7); };
        auto look = [&](int which, int j) {
            return &s_look[((which * kLookRing + (j & (kLookRing - 1))) * kWaves + wave) * kTokPerWave];
        };
        auto sp_issue_pos = [&](int j) {           // slots past the row: its last entry
            if (lane < kTokPerWave)
                lds_dma_glb4(indices + (int64_t)b * a.topk + min(sp_slot(j), a.topk - 1), lds_addr(look(0, j)));
        };
        auto sp_issue_page = [&](int j, int pos) { // no real token: the row's first page
            const bool ok = sp_slot(j) < t1 && pos >= 0 && pos < Lb;
            if (lane < kTokPerWave)
                lds_dma_glb4(bt + (int64_t)b * a.max_pages + (ok ? pos >> a.page_shift : 0), lds_addr(look(1, j)));
        };
        auto sp_read = [&](int which, int j) {     // a lookup that is in; lane l: token l % 8
            int v;
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v)
                         : "v"(lds_addr(look(which, j)) + 4 * (lane & 7)) : "memory");
            return v;
        };

        // ---- loads of tile t into its ring slot: token tt of the wave (tile row 8 wave +
        //      tt) by lanes 0-40 through a buffer resource over that token's 656 bytes, or
        //      over none (reads as zeros) when it is not real.  Sparse: the page ids of tile
        //      t + kAhead and the positions of tile t + 2 kAhead go out first; the lookups
        //      this uses were loaded kAhead tiles ago.
        // dense: page id of the wave's first token of the next tile to load (tile 0 here)
        int next_page = SPARSE ? 0 : bt[(int64_t)b * a.max_pages + (min(t0 + kTokPerWave * wave, t1 - 1) >> a.page_shift)];
        auto issue_tile = [&](int t) {
            uint8_t *dst = &raw[t % kRawSlots][kTokPerWave * wave * kRawRow];
            if (SPARSE) {
                const int pos_look = sp_read(0, t + kAhead);
                sp_issue_page(t + kAhead, pos_look);
                sp_issue_pos(t + 2 * kAhead);
                const int pos = sp_read(0, t), page = sp_read(1, t);
                uint32_t vm = 0;
#pragma unroll
                for (int tt = 0; tt < kTokPerWave; tt++) {
                    const int p = __builtin_amdgcn_readlane(pos, tt);
                    const int pg = __builtin_amdgcn_readlane(page, tt);
                    const int k = t0 + kT * t + kTokPerWave * wave + tt;
                    const bool ok = k < t1 && p >= 0 && p < Lb;
                    vm |= (ok ? 1u : 0u) << tt;
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                        (void *)(a.k_pool + (ok ? (int64_t)pg * a.s_page_b + (int64_t)(p & page_mask) * a.s_tok_b : 0)),
                        (short)0, ok ? kTokBytes : 0, 0x00020000);
                    if (lane < kChunks) lds_dma_buf16(rs, 16 * lane, lds_addr(dst + tt * kRawRow));
                }
                if (lane == 0) ((uint8_t *)&s_valid[t % kRawSlots])[wave] = (uint8_t)vm;
            } else {
                const int tw = t0 + kT * t + kTokPerWave * wave;     // first of the 8 tokens
                const int page = next_page;
                // the next tile's page id, loaded now and used one tile later
                next_page = bt[(int64_t)b * a.max_pages + (min(tw + kT, t1 - 1) >> a.page_shift)];
                // the 8 tokens are consecutive slots of one page: one 64-bit address, then
                // one stride step per token
                const uint8_t *tok = a.k_pool + (int64_t)page * a.s_page_b + (int64_t)(tw & page_mask) * a.s_tok_b;
                const int nreal = min(max(t1 - tw, 0), kTokPerWave);
                const uint32_t lds0 = lds_addr(dst);
#pragma unroll
                for (int tt = 0; tt < kTokPerWave; tt++) {
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                        (void *)tok, (short)0, tt < nreal ? kTokBytes : 0, 0x00020000);
                    if (lane < kChunks) lds_dma_buf16(rs, 16 * lane, lds0 + tt * kRawRow);
                    tok += a.s_tok_b;
                }
            }
        };

        // ---- Q^T operand of this wave's 16 heads (B of the MFMAs), resident.  Latent dims:
        //      for each 128-dim tile u, an fp8 pair q = hi 2^e_hi + lo 2^e_lo (power-of-two
        //      scales per head and tile, taken by the scaled MFMA), so the K codes enter the
        //      MFMA as they are; lane (col, g4) holds dims 128u + 16g4 + 0..15 (bytes 0-15)
        //      and 128u + 64 + 16g4 + 0..15 (bytes 16-31), the k order of the fp8 MFMA.  Rope
        //      dims stay bf16: step r <- dims 512 + 32r + 8g4 .. +7.  A wave with no query
        //      rows runs the same instruction stream on a zero Q; it writes nothing.
        i32x8 qhi[4], qlo[4];
        uint32_t qsc_hi = 0x7F7F7F7Fu, qsc_lo = 0x7F7F7F7Fu;   // E8M0 byte u: tile u
        bf16x8 qrope[2];
        {
            const uint16_t *qrow = a.q + (((int64_t)b * nq + qi) * Hq + head0 + col) * kDqk;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                float v[32];
                u32x4 raw4[4];
#pragma unroll
                for (int h = 0; h < 4; h++)
                    raw4[h] = active ? *(const u32x4 *)(qrow + 128 * u + 64 * (h >> 1) + 16 * g4 + 8 * (h & 1))
                                     : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const uint32_t w2 = raw4[i >> 2][i & 3];
                    v[2 * i] = __uint_as_float(w2 << 16);
                    v[2 * i + 1] = __uint_as_float(w2 & 0xFFFF0000u);
                }
                const int e_hi = q_split_exp(v);
                const int e_lo = q_split_lo(v, e_hi, qhi[u], qlo[u]);
                qsc_hi = (qsc_hi & ~(0xFFu << (8 * u))) | ((uint32_t)(127 + e_hi) << (8 * u));
                qsc_lo = (qsc_lo & ~(0xFFu << (8 * u))) | ((uint32_t)(127 + e_lo) << (8 * u));
            }
#pragma unroll
            for (int r = 0; r < 2; r++)
                qrope[r] = active ? *(const bf16x8 *)(qrow + 512 + 32 * r + 8 * g4) : bf16x8{};
        }

        f32x4 acc[kDvBlocks];
#pragma unroll
        for (int i = 0; i < kDvBlocks; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY;     // reference max (log2 domain) of head `col`
        float l = 0.f;

        // ---- S^T of tile t (rows: this lane's tokens 8g4 + 4sb + r, r = 0..3): one partial
        //      per 128-dim scale tile (two scaled fp8 MFMAs 16x16x128: Q's hi and lo terms)
        //      and one for the rope dims (two bf16 MFMAs 16x16x32), combined with the token
        //      scales in fp32.  inter(k) runs right after MFMA slot k (k = 0..19), with
        //      nothing moved across it.
        auto qk_tile = [&](int t, float (&st)[8], auto &&inter) {
            const uint8_t *slot = raw[t % kRawSlots];
#pragma unroll
            for (int sb = 0; sb < 2; sb++) {
                f32x4 part[5];
#pragma unroll
                for (int p = 0; p < 5; p++) part[p] = f32x4{0.f, 0.f, 0.f, 0.f};
                const uint8_t *kbase = slot + qk_off0 + 4 * sb * kRawRow;
                // the 32 code bytes of tile u in the fp8 MFMA's k order
                auto rd_codes = [&](int u) {
                    const u32x4 x = *(const u32x4 *)(kbase + 128 * u);
                    const u32x4 y = *(const u32x4 *)(kbase + 128 * u + 64);
                    return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
                };
                auto rd_rope = [&](int r) { return *(const bf16x8 *)(kbase + 512 + 16 + 64 * r); };
                i32x8 kc[4];
                bf16x8 kr[2];
                kc[0] = rd_codes(0);
                kc[1] = rd_codes(1);
                // slot k: tiles (0, 1) hi, (0, 1) lo, (2, 3) hi, (2, 3) lo, rope 0, 1; each
                // read is issued two slots or more before its first use
#pragma unroll
                for (int k = 0; k < 10; k++) {
                    if (k == 0) kc[2] = rd_codes(2);
                    if (k == 1) kc[3] = rd_codes(3);
                    if (k == 4) kr[0] = rd_rope(0);
                    if (k == 5) kr[1] = rd_rope(1);
                    if (k < 8) {
                        const int u = 2 * (k >> 2) + (k & 1);
                        const bool lo = (k & 2) != 0;
                        part[u] = mfma_fp8_q(u, kc[u], lo ? qlo[u] : qhi[u], part[u], lo ? qsc_lo : qsc_hi);
                    } else {
                        part[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[k - 8], qrope[k - 8], part[4], 0, 0, 0);
                    }
                    inter(10 * sb + k);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const f32x4 sc = *(const f32x4 *)(slot + sc_off + (4 * sb + r) * kRawRow);
                    float x = part[4][r];
#pragma unroll
                    for (int p = 0; p < 4; p++) x += sc[p] * part[p][r];
                    st[4 * sb + r] = x;
                }
            }
        };

        // ---- softmax of tile j (S^T in st) in steps, k = 0..kSmSteps-1: logits and mask,
        //      the max over the head's 32 tokens, the lazily moved reference m_new,
        //      p = 2^(s - m_new) and their sum ps
        float sv[8], bm = -INFINITY, m_new = m, pr[8], ps = 0.f;
        auto sm_step = [&](int j, const float (&st)[8], int k) {
            switch (k) {
            case 0: {
                const uint32_t vmask = SPARSE ? s_valid[j % kRawSlots] : 0u;
                bm = -INFINITY;
#pragma unroll
                for (int r = 0; r < 8; r++) {
                    const int row = 8 * g4 + r;                 // token within the tile
                    const int tok = t0 + kT * j + row;
                    const bool vis = SPARSE ? ((vmask >> row) & 1u) != 0
                                            : MASKED ? (tok < tlim && tok >= tlo) : tok < t1;
                    sv[r] = vis ? st[r] * a.scale_log2 : -INFINITY;
                    bm = fmaxf(bm, sv[r]);
                }
                break;
            }
            case 2:
                bm = col_max(bm);
                m_new = bm > m + kLazyMax ? bm : m;
                break;
            case 4:
            case 6: {
                const float mref = m_new == -INFINITY ? 0.f : m_new;
                const int r0 = k == 4 ? 0 : 4;
#pragma unroll
                for (int r = r0; r < r0 + 4; r++) {
                    pr[r] = fast_exp2(sv[r] - mref);
                    asm volatile("" : "+v"(pr[r]));       // computed here, not after the branch
                }
                break;
            }
            case 8:
                ps = 0.f;
#pragma unroll
                for (int r = 0; r < 8; r++) ps += pr[r];
                break;
            default:
                break;
            }
        };
        constexpr int kSmSteps = 9;

        // ---- O^T += V^T . P^T for tile j: A = V^T from the transposed code read (this
        //      lane: value dim 16db + col, tokens 8g4 + 0..7), B = P^T times the value
        //      tile's token scales (pbt[t], built 3 MFMAs before MFMA 8t from scales read
        //      4 MFMAs before that)
        auto pv_tile = [&](int j) {
            const uint8_t *slot = raw[j % kRawSlots];
            const uint8_t *vbase = slot + pv_off;
            bf16x8 pbt[4];
            float scv[8];
            auto scale_read = [&](int t) {         // tile t's scales of this lane's 8 tokens
#pragma unroll
                for (int r = 0; r < 8; r++) scv[r] = *(const float *)(slot + sc_off + r * kRawRow + 4 * t);
            };
            auto p_times_scale = [&](int t) {
#pragma unroll
                for (int r = 0; r < 8; r++) pbt[t][r] = (__bf16)(pr[r] * scv[r]);
            };
            auto rd = [&](int db) {
                return __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2 *)(PA_LDS uint8_t *)(vbase + 16 * db));
            };
            i32x2 vw[3];
            scale_read(0);
            vw[0] = rd(0);
            vw[1] = rd(1);
            p_times_scale(0);
            bf16x8 va[2];
            va[0] = fp8x8_to_bf16((uint32_t)vw[0][0], (uint32_t)vw[0][1]);
#pragma unroll
            for (int db = 0; db < kDvBlocks; db++) {
                if (db + 2 < kDvBlocks) vw[(db + 2) % 3] = rd(db + 2);
                acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db & 1], pbt[db >> 3], acc[db], 0, 0, 0);
                if (db + 1 < kDvBlocks)
                    va[(db + 1) & 1] = fp8x8_to_bf16((uint32_t)vw[(db + 1) % 3][0], (uint32_t)vw[(db + 1) % 3][1]);
                if ((db & 7) == 1 && db < 24) scale_read((db >> 3) + 1);
                if ((db & 7) == 5 && db < 24) p_times_scale((db >> 3) + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        if (ntiles > 0) {
            // ---- prologue: lookups (sparse), the loads of tiles 0..kRawSlots-2, S^T of
            //      tile 0
            if (SPARSE) {
                for (int t = 0; t < 2 * kAhead; t++) sp_issue_pos(t);
                wait_vmcnt<0>();
                for (int t = 0; t < kAhead; t++) sp_issue_page(t, sp_read(0, t));
                wait_vmcnt<0>();
            }
#pragma unroll
            for (int t = 0; t < kRawSlots - 1; t++) {
                // tile t's lookups came from tile t - kAhead's loads
                if (SPARSE && t >= kAhead) wait_vmcnt<(kAhead - 1) * kLoadsPerTile>();
                issue_tile(t);
            }
            wait_vmcnt<(kRawSlots - 2) * kLoadsPerTile>();   // tile 0 in
            lds_barrier();

            float st[8], st_next[8];
            qk_tile(0, st, [](int) {});

            // The tile loop never rescales O^T itself: when a tile's max exceeds the
            // reference by more than 2^8 it leaves after phase 1, the rescale runs outside,
            // and the loop redoes phase 1 of the same tile with the new reference.  Inside
            // the loop O^T is only touched by MFMAs, so it stays in the accumulation
            // registers.
            int j = 0;
            bool redo = false;
            for (;;) {
            for (; j < ntiles; j++) {
                if (!redo) {
                    // ---- top: tile j+1's loads in (tiles j+2.. are younger), all waves
                    //      past tile j-1, then tile j+kRawSlots-1's loads into its slot
                    wait_vmcnt<(kRawSlots - 3) * kLoadsPerTile>();
                    lds_barrier();
                    issue_tile(j + kRawSlots - 1);
                }
                redo = false;
                // ---- phase 1: QK of tile j+1 (after the last tile: a dummy on the next
                //      slot), the softmax of tile j between its MFMAs
                qk_tile(j + 1, st_next, [&](int k) {
                    if (k < kSmSteps) sm_step(j, st, k);
                });
                if (__any(m_new != m)) break;
                l += ps;
                // ---- phase 2: PV of tile j
                pv_tile(j);
#pragma unroll
                for (int r = 0; r < 8; r++) st[r] = st_next[r];
            }
            if (j >= ntiles) break;
            // move the reference to m_new and rescale (rare; every item's first tile).
            // The multiply reads and writes O^T in place, so it stays in the accumulation
            // registers (a plain multiply would make the compiler copy all of O^T out).
            {
                const float alpha = fast_exp2(m - m_new);    // m = -inf: 0
                m = m_new;
                l = l * alpha;
#pragma unroll
                for (int i = 0; i < kDvBlocks; i++) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        float v = acc[i][e], tmp;
                        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                                     : "+a"(v), "=&v"(tmp) : "v"(alpha));
                        acc[i][e] = v;
                    }
                }
                redo = true;
            }
            }
            wait_vmcnt<0>();
        }

        // ---- epilogue: this wave's heads are complete for this item
        if (active) {
            l = col_sum(l);
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
