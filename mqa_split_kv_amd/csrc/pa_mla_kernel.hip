// Split-KV MQA decode over the MLA 656-byte FP8 latent cache (D_qk = 576, D_v = 512,
// one KV head shared by G query heads, G a multiple of 16 up to 128), gfx950.
//
// Token layout (FlashMLA walk-through, section 数据加载, byte-layout table): 512 e4m3
// codes, 4 fp32 scales (one per 128 codes), 64 bf16 rope values.  The key is the 576
// dequantised values, the value is their first 512 (V shares the latent with K).
//
// One workgroup (8 waves, two per SIMD) = one (part, group of 64 query rows); it walks
// the part's items.  Query rows are (draft token qi, head g) pairs, row qi * G + g, so with
// several query tokens per request (a linear speculative draft) each block of 16 rows
// shares one draft token and its causal limit L - q_len + qi + 1.  The two head groups of a
// part run as workgroups 8 ids apart, i.e. on the same XCD at about the same time, so the
// second read of each KV tile is an L2 hit (the FlashMLA walk-through shares one KV tile
// between two 64-head CTAs through a cluster, section 计算环节一; here the L2 of the XCD
// plays that role).
//
// Waves hg and hg + 4 share a SIMD, with two roles (the FlashMLA walk-through splits a
// tile's work over two warpgroups, section 计算环节二; here the split is by operation):
//   * score wave hg (Q of head block hg resident) computes S^T[32 tok x 16 heads] = K . Q^T;
//     in iteration i it runs tile i+1's MFMAs and, between them, tile i's softmax, and hands
//     P^T of tile i to the value waves through LDS;
//   * value wave hg (O^T of value dims 128 hg .. +127 for all 64 heads resident, 128
//     registers) runs O^T += V^T . P^T of tile i-1 in iteration i: each V^T operand is read
//     and converted once and feeds the 4 head blocks' MFMAs.
// Two waves per SIMD let one wave's conversions, softmax and waits run under the other's
// matrix work; the score wave also overlaps its own softmax with its next tile's MFMAs (a
// wave's dependent VALU chains and its LDS and barrier waits otherwise stall its own MFMA
// issue).
//
// Per 32-token tile:
//   * the tokens' 656 bytes go HBM -> LDS by direct-to-LDS loads (one instruction per
//     token, 41 lanes of 16 bytes; a token that is not real reads as zeros) into a 5-slot
//     ring of 752-byte rows (the stride at which both operand read patterns below run at
//     the LDS's measured best); tile i+3's loads go out at the top of iteration i, after
//     the wait for tiles i and i+1 (the score waves read tile i+1's keys).  Page ids
//     come the same way, 3 tiles ahead, into a small LDS ring (a scalar load would make
//     every later LDS wait also wait for it);
//   * scores: the FP8 codes enter a scaled fp8 MFMA 16x16x128 as they are; Q is resident as
//     two e4m3 terms with power-of-two scales per head and tile (q = hi 2^e_hi + lo 2^e_lo,
//     exact to 2^-21 of the tile's max), so each 128-dim tile is two MFMAs.  The rope dims
//     use bf16 MFMA 16x16x32.  The token scales are applied in fp32 to the per-tile
//     partials: S = sum_t scale_t (q_t . k_t) + q_rope . k_rope.  (The FlashMLA walk-through
//     dequantises to bf16 and runs bf16 MMA with fp32 accumulation, section 计算环节一; here
//     no operand of the score product is converted.)
//   * an online softmax per head column (the previous tile's, in the MFMA slots of the next
//     tile's scores); the score wave writes P^T times each 128-dim value tile's token scales
//     (bf16, the B operands of the PV MFMAs) and the factor for O^T (1 unless the reference
//     max moved);
//   * O^T += V^T . P^T with bf16 MFMA 16x16x32, V^T read transposed from the FP8 codes
//     (ds_read_b64_tr_b8) and converted in registers (exact).  O^T takes 128 registers (the
//     register-budget problem the FlashMLA walk-through describes in section 计算环节二),
//     ordinary VGPRs: one kernel has one split between VGPRs and accumulation registers,
//     and the score wave's registers are VGPRs.
// Operand layouts.  QK row block sb (0, 1) of the A operand holds, in MFMA row m = 4g + r,
// token 8g + 4sb + r, so lane group g of the S^T result holds tokens 8g..8g+7: exactly the
// k slots the same lanes of a value wave feed to the PV MFMA (B = P^T, k = 8g + j), and
// the transposed read returns tokens 8g..8g+7 of one value dim per lane; the PV operands
// pass through LDS lane for lane.  In the fp8 MFMA lane (col, g) holds dims 16g + 0..15
// and 64 + 16g + 0..15 of the 128-dim tile.
// One workgroup barrier per tile: it publishes the PV operands of tile i-1 and frees the
// ring slot of tile i-2.  The running max is only moved when a tile's max exceeds it by
// more than 2^8, so the rescale of O^T is rare; probabilities stay below 2^8 and the result
// is the same up to rounding (the reference cancels in the final normalisation).
//
// Sparse decode (FlashMLA walk-through, section 调度: the decode call takes sparse
// indices): the items then cover index slots, and slot k of request b names the key
// position indices[b][k].  The address of a listed token takes two dependent lookups
// (index, then block table); lanes 0-3 of each wave (its 4 tokens of a tile) load them
// direct to LDS, positions 6 tiles and page ids 3 tiles ahead of the tile's own loads,
// so that every wait for them is one the KV ring does anyway.  A slot outside the item or
// the request loads nothing (zeros), and a per-tile bit mask of the real tokens is
// applied in the softmax.
#include "pa_internal.h"
#include "pa_merge.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define PA_LDS __attribute__((address_space(3)))

constexpr int kWaves = 8;                          // 4 score waves, then 4 value waves
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = kWaves / 2 * kHeadsPerWave;   // 64
constexpr int kDqk = 576, kDv = 512;
constexpr int kTokBytes = 656;
constexpr int kChunks = kTokBytes / 16;            // 41 16-byte chunks per token
constexpr int kT = 32;                             // tokens per tile
constexpr int kTokPerWave = kT / kWaves;           // 4 tokens loaded per wave and tile
constexpr int kRawRow = 752;                       // LDS row of a token (656 + 96)
constexpr int kRawTile = kT * kRawRow;             // 24064
constexpr int kRawSlots = 5;                       // tile ring
constexpr int kAhead = kRawSlots - 2;              // loads go out 3 tiles ahead (2 ahead of the keys'
                                                   // first use); lookups: page ids 3 (sparse:
                                                   // positions 6) tiles ahead
constexpr int kLookRing = 8;                       // lookup slots (tiles) per wave
constexpr int kDvBlocks = kDv / 16;                // O^T blocks of a value wave (8 dims x 4 heads), 32 MFMAs a tile
constexpr int kVBlocks = 128 / 16;                 // 16-dim blocks of a value wave's value tile
constexpr float kLazyMax = 8.0f;                   // log2 units

static_assert(kRawSlots >= 4, "the tile loop reads tiles i and i-1 with loads in flight");
static_assert(kLookRing > 2 * kAhead && (kLookRing & (kLookRing - 1)) == 0, "lookup ring");

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool SPARSE>
struct MlaCfg {
    // loads per wave and tile: one per token, one page-id load (sparse: plus one index load)
    static constexpr int kLoadsPerTile = SPARSE ? kTokPerWave + 2 : kTokPerWave + 1;
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
// every wait for them in this file is explicit.  Nothing else here uses M0.  The scalar
// operands (the buffer over `nbytes` bytes at `base`, the LDS address) are made uniform
// explicitly: the asm takes them in scalar registers.
__device__ __forceinline__ void lds_dma_buf16(const void *base, int nbytes, int voff, uint32_t lds)
{
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint64_t pu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(uintptr_t)pu, (short)0, __builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma_glb4(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g) : "memory", "m0");
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

// O^T += A B in place, as inline asm: the accumulator is tied to its registers (with the
// builtin the compiler may rename O^T's blocks from one tile to the next and copy them
// back at the loop edge, 4 cycles per register), and they are ordinary VGPRs: one
// kernel has one split between VGPRs and accumulation registers, and the score waves'
// registers are VGPRs.  The compiler does not see into the asm: a VALU write of A, B or
// the accumulator must be at least 2 instructions before it (the callers convert A two
// MFMAs ahead), and every VALU read of O^T after the last of these MFMAs follows
// mfma_acc_drain().
__device__ __forceinline__ void mfma_acc(f32x4 &acc, const bf16x8 &a, const bf16x8 &b)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// The drain waits out the MFMA latency and redefines every accumulator through the asm,
// so no read of O^T can be placed above it.
template <int N>
__device__ __forceinline__ void mfma_acc_drain(f32x4 (&acc)[N])
{
    static_assert(N % 8 == 0, "drain in groups of 8");
    asm volatile("s_nop 15\n\ts_nop 15" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]),
                 "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7]));
#pragma unroll
    for (int g = 8; g < N; g += 8)
        asm volatile("" : "+v"(acc[g]), "+v"(acc[g + 1]), "+v"(acc[g + 2]), "+v"(acc[g + 3]),
                     "+v"(acc[g + 4]), "+v"(acc[g + 5]), "+v"(acc[g + 6]), "+v"(acc[g + 7]));
}

// SPARSE: index-slot items.  MASKED: a per-head-block key range narrower than the item
// (draft tokens' causal limits, a sliding window); separate instantiations keep the plain
// kernel's registers free.
template <bool SPARSE, bool MASKED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void pa_mla_kernel(
    DecodeArgs a, const int32_t *__restrict__ plan, const int32_t *__restrict__ bt, int ngroups,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ indices)
{
    constexpr int kLoadsPerTile = MlaCfg<SPARSE>::kLoadsPerTile;
    __shared__ __attribute__((aligned(16))) uint8_t raw[kRawSlots][kRawTile];
    // the PV B operands of a tile from the score wave of head block hg, in its lanes' layout
    // (lane (col, g4): head col, tokens 8g4 + 0..7): P^T times value tile t's token scales,
    // bf16: [tile parity][hg][value tile t][lane]
    __shared__ bf16x8 s_p[2][4][4][64];
    __shared__ float s_alpha[2][4][16];       // factor on O^T before the tile's PV, per head
    __shared__ float s_inv[4][16];            // the item's final 1 / l, per head
    __shared__ int s_flag;                    // fused combine: this workgroup merges
    __shared__ __attribute__((aligned(4))) uint8_t s_valid[kRawSlots][kWaves];   // sparse: real-token bits
    // lookups: [position | page id][tile % kLookRing][wave][token] (dense: page ids of the
    // wave's first token only)
    __shared__ int32_t s_look[2 * kLookRing * kWaves * kTokPerWave];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int hg = wave & 3;                       // score: head block; value: value tile (same SIMD)
    const bool scorer = wave < 4;                  // score wave; else value wave
    // workgroup id -> (part, head group): the head groups of one part are 8 ids apart
    const int wg = blockIdx.x;
    const int part = (wg / (8 * ngroups)) * 8 + wg % 8;
    const int group = (wg / 8) % ngroups;
    if (part >= a.num_parts) return;               // padding of the last id block
    const int G = a.G, Hq = a.Hkv * a.G, nq = a.q_len;
    const int row0 = group * kHeadsPerWG + hg * kHeadsPerWave;     // first query row
    const bool active = row0 < G * nq;             // wave-uniform
    const int qi = row0 / G;                       // the block's draft token (G % 16 == 0)
    const int head0 = row0 - qi * G;               // its first head
    const int col = lane & 15, g4 = lane >> 4;     // MFMA column (head), lane group
    const int page_mask = (1 << a.page_shift) - 1;

    // LDS byte offsets inside a tile slot: the QK operand rows of row block 0 (token
    // 8(col/4) + col%4 at this lane's 16 bytes of each 64-dim group; row block 1 is 4 rows
    // further), the rope operand, the scale rows of this lane's tokens 8g4 + r, and the
    // transposed PV read (lane pair 2r, 2r+1 of a 16-lane block supplies row 8g4 + r,
    // bytes 0-7 and 8-15 of the block's 16 value dims)
    const uint32_t qk_off = (uint32_t)((8 * (col >> 2) + (col & 3)) * kRawRow + 16 * g4);
    const uint32_t rope_off = qk_off + 528;
    const uint32_t sc_off = (uint32_t)(8 * g4 * kRawRow + 512);
    const uint32_t pv_off = (uint32_t)((8 * g4 + ((lane & 15) >> 1)) * kRawRow + 8 * (lane & 1));

    // a fixed-split plan has exactly one item per part (no plan read on the critical path)
    const int ib = a.fixed_splits > 0 ? part : plan[a.part_begin_off + part];
    const int ie = a.fixed_splits > 0 ? part + 1 : plan[a.part_begin_off + part + 1];

    for (int it = ib; it < ie; it++) {
        const int b = plan[a.items_off + 4 * it + 0];
        const int t0 = plan[a.items_off + 4 * it + 1];
        const int t1 = plan[a.items_off + 4 * it + 2];
        const int flags = plan[a.items_off + 4 * it + 3];
        const int ntiles = (t1 - t0 + kT - 1) / kT;
        const int64_t qr = (int64_t)qi * Hq + head0 + col;     // query row within the request

        // ---- lookups.  Sparse: lane l < 4 loads those of token l of the wave's 4 in tile j,
        //      index slot k.  Dense: lane 0 loads the page id of the wave's first token of
        //      tile j (its 4 tokens are consecutive slots of one page).
        const int Lb = SPARSE ? seq_lens[b] : 0;
        auto sp_slot = [&](int j) { return t0 + kT * j + kTokPerWave * wave + (lane & (kTokPerWave - 1)); };
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
        auto sp_read = [&](int which, int j) {     // a lookup that is in; lane l: token l % 4
            int v;
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v)
                         : "v"(lds_addr(look(which, j)) + 4 * (lane & (kTokPerWave - 1))) : "memory");
            return v;
        };
        auto dn_issue_page = [&](int j) {          // past the item: its last token's page
            if (lane == 0)
                lds_dma_glb4(bt + (int64_t)b * a.max_pages + (min(t0 + kT * j + kTokPerWave * wave, t1 - 1) >> a.page_shift),
                             lds_addr(look(1, j)));
        };
        // dense: the page id of tile t (uniform), read from LDS; the value exists only after
        // its wait, inside the same asm statement (an intrinsic on the loaded register could
        // be moved above a separate wait).  page_barrier also does the loop top's barrier,
        // with the read in flight across it.
        auto dn_page = [&](int t) {
            int v, pg;
            asm volatile("ds_read_b32 %0, %2\n\ts_waitcnt lgkmcnt(0)\n\tv_readfirstlane_b32 %1, %0"
                         : "=&v"(v), "=s"(pg) : "v"(lds_addr(look(1, t))) : "memory");
            return pg;
        };
        auto page_barrier = [&](int t) {
            int v, pg;
            asm volatile("s_waitcnt lgkmcnt(0)\n\tds_read_b32 %0, %2\n\ts_barrier\n\ts_waitcnt lgkmcnt(0)\n\t"
                         "v_readfirstlane_b32 %1, %0"
                         : "=&v"(v), "=s"(pg) : "v"(lds_addr(look(1, t))) : "memory");
            return pg;
        };

        // ---- loads of tile t into its ring slot: token tt of the wave (tile row 4 wave + tt)
        //      by lanes 0-40 through a buffer over that token's 656 bytes, or over none (reads
        //      as zeros) when it is not real.  Sparse: the page ids of tile t + kAhead and the
        //      positions of tile t + 2 kAhead go out first; the lookups this uses were loaded
        //      kAhead tiles ago.  Dense: the page id of tile t + kAhead goes out last.
        auto issue_tile = [&](int t, int page) {
            uint8_t *dst = &raw[t % kRawSlots][kTokPerWave * wave * kRawRow];
            if (SPARSE) {
                const int pos_look = sp_read(0, t + kAhead);
                sp_issue_page(t + kAhead, pos_look);
                sp_issue_pos(t + 2 * kAhead);
                const int pos = sp_read(0, t), pgv = sp_read(1, t);
                uint32_t vm = 0;
#pragma unroll
                for (int tt = 0; tt < kTokPerWave; tt++) {
                    const int p = __builtin_amdgcn_readlane(pos, tt);
                    const int pg = __builtin_amdgcn_readlane(pgv, tt);
                    const int k = t0 + kT * t + kTokPerWave * wave + tt;
                    const bool ok = k < t1 && p >= 0 && p < Lb;
                    vm |= (ok ? 1u : 0u) << tt;
                    const uint8_t *src = a.k_pool + (ok ? (int64_t)pg * a.s_page_b + (int64_t)(p & page_mask) * a.s_tok_b : 0);
                    if (lane < kChunks) lds_dma_buf16(src, ok ? kTokBytes : 0, 16 * lane, lds_addr(dst + tt * kRawRow));
                }
                if (lane == 0) s_valid[t % kRawSlots][wave] = (uint8_t)vm;
            } else {
                // the 4 tokens are consecutive slots of one page
                const int tw = t0 + kT * t + kTokPerWave * wave;     // first of the 4 tokens
                const uint8_t *tok = a.k_pool + (int64_t)page * a.s_page_b + (int64_t)(tw & page_mask) * a.s_tok_b;
                const int nreal = min(max(t1 - tw, 0), kTokPerWave);
                const uint32_t lds0 = lds_addr(dst);
#pragma unroll
                for (int tt = 0; tt < kTokPerWave; tt++)
                    if (lane < kChunks)
                        lds_dma_buf16(tok + (int64_t)tt * a.s_tok_b, tt < nreal ? kTokBytes : 0, 16 * lane, lds0 + tt * kRawRow);
                dn_issue_page(t + kAhead);
            }
        };

        // ---- top of tile i (both roles, same barriers): tile i's loads in (tiles i+1 ..
        //      i+kAhead-1 are younger), all waves past tile i-1 (slot of tile i-2 free, the
        //      B operands of tile i-1 stored), then tile i+kAhead's loads into its slot (every
        //      wave issues exactly one tile's loads per iteration, which the wait counts rely
        //      on; issued here or spread between the MFMAs measured the same)
        auto tile_top = [&](int i) {
            wait_vmcnt<(kAhead - 2) * kLoadsPerTile>();
            if (SPARSE) {
                lds_barrier();
                issue_tile(i + kAhead, 0);
            } else {
                issue_tile(i + kAhead, page_barrier(i + kAhead));
            }
        };

        if (ntiles > 0) {
            // ---- prologue: lookups (sparse), the loads of tiles 0..kAhead-1
            if (SPARSE) {
                for (int t = 0; t < 2 * kAhead; t++) sp_issue_pos(t);
                wait_vmcnt<0>();
                for (int t = 0; t < kAhead; t++) sp_issue_page(t, sp_read(0, t));
            } else {
                for (int t = 0; t < kAhead; t++) dn_issue_page(t);
            }
            wait_vmcnt<0>();
#pragma unroll
            for (int t = 0; t < kAhead; t++) issue_tile(t, SPARSE ? 0 : dn_page(t));
        }

        if (scorer) {
            // ================= score wave: S, softmax and P of tile i in iteration i
            // causal limit of the block's draft token and the first key its window leaves
            int tlim = t1, tlo = 0;
            if (MASKED) {
                const int L = seq_lens[b];
                if (nq > 1) tlim = min(t1, L - (nq - 1 - qi));
                if (a.window > 0) tlo = max(0, L - nq + qi - a.window + 1);
            }
            // Q^T of the block's 16 heads (B of the MFMAs), resident.  Latent tile u: an fp8
            // pair per head, lane (col, g4) holding dims 128u + 16g4 + 0..15 (bytes 0-15) and
            // 128u + 64 + 16g4 + 0..15 (bytes 16-31), the k order of the fp8 MFMA.  Rope: bf16,
            // step r <- dims 512 + 32r + 8g4 .. +7.  A block with no query rows runs on a zero
            // Q and writes nothing.
            i32x8 qhi[4], qlo[4];
            uint32_t qsc_hi = 0, qsc_lo = 0;          // E8M0 byte u: tile u
            bf16x8 qrope[2];
            {
                const uint16_t *qrow = a.q + ((int64_t)b * nq * Hq + qr) * kDqk;
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    float v[32];
                    u32x4 raw4[4];
#pragma unroll
                    for (int h = 0; h < 4; h++)
                        raw4[h] = active ? *(const u32x4 *)(qrow + 128 * u + 64 * (h >> 1) + 16 * g4 + 8 * (h & 1))
                                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int x = 0; x < 16; x++) {
                        const uint32_t w2 = raw4[x >> 2][x & 3];
                        v[2 * x] = __uint_as_float(w2 << 16);
                        v[2 * x + 1] = __uint_as_float(w2 & 0xFFFF0000u);
                    }
                    const int e_hi = q_split_exp(v);
                    const int e_lo = q_split_lo(v, e_hi, qhi[u], qlo[u]);
                    qsc_hi |= (uint32_t)(127 + e_hi) << (8 * u);
                    qsc_lo |= (uint32_t)(127 + e_lo) << (8 * u);
                }
#pragma unroll
                for (int r = 0; r < 2; r++)
                    qrope[r] = active ? *(const bf16x8 *)(qrow + 512 + 32 * r + 8 * g4) : bf16x8{};
            }
            float m = -INFINITY;     // reference max (log2 domain) of head `col`
            float l = 0.f;

            // ---- S^T of tile t (rows: this lane's tokens 8g4 + 4sb + r) into st[8]: one partial
            //      per 128-dim scale tile u (two scaled fp8 MFMAs 16x16x128, Q's hi and lo
            //      terms) and one for the rope dims (two bf16 MFMAs 16x16x32), combined with
            //      the token scales in fp32 as each pair of tiles completes.  MFMA slot k of row
            //      block sb: rope 0, 1, tiles (0,1) hi, (0,1) lo, (2,3) hi, (2,3) lo; every
            //      operand is read two slots before its first use.  step(s) runs in slot
            //      s = 10 sb + k, before its MFMA: the VALU work of the previous tile, issued
            //      while the matrix core works (and, first, while the tile's first reads
            //      are on their way).
            auto qk_tile = [&](int t, float (&st)[8], auto &&step) {
                PA_LDS const uint8_t *slot = (PA_LDS const uint8_t *)raw[t % kRawSlots];
                auto rd_codes = [&](int sb, int u) {
                    PA_LDS const uint8_t *p = slot + qk_off + 4 * sb * kRawRow + 128 * u;
                    const u32x4 x = *(PA_LDS const u32x4 *)p;
                    const u32x4 y = *(PA_LDS const u32x4 *)(p + 64);
                    return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
                };
                auto rd_rope = [&](int sb, int r) { return *(PA_LDS const bf16x8 *)(slot + rope_off + 4 * sb * kRawRow + 64 * r); };
                i32x8 kc[2][4];
                bf16x8 kr[2][2];
                f32x4 part[2][5];
                f32x4 sc[8];                       // token 8g4 + r's four tile scales
                kr[0][0] = rd_rope(0, 0);
                kr[0][1] = rd_rope(0, 1);
                // rows 2h, 2h+1 of row block sb, tiles 2v and 2v+1: the token scales times the
                // tile partials, added to the rope partial (v = 0) or the sum so far (v = 1)
                auto combine = [&](int sb, int v, int h) {
#pragma unroll
                    for (int r = 2 * h; r < 2 * h + 2; r++) {
                        float x = v == 0 ? part[sb][4][r] : st[4 * sb + r];
#pragma unroll
                        for (int u = 2 * v; u < 2 * v + 2; u++) x += sc[4 * sb + r][u] * part[sb][u][r];
                        asm volatile("" : "+v"(x));    // computed in this slot
                        st[4 * sb + r] = x;
                    }
                };
#pragma unroll
                for (int sb = 0; sb < 2; sb++) {
#pragma unroll
                    for (int p = 0; p < 5; p++) part[sb][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < 10; k++) {
                        // reads issued at this slot (the token scales early, for the combine)
                        if (k == 0) kc[sb][0] = rd_codes(sb, 0);
                        if (k == 1) kc[sb][1] = rd_codes(sb, 1);
                        if (k >= 2 && k < 6)
                            sc[4 * sb + k - 2] = *(PA_LDS const f32x4 *)(slot + sc_off + (4 * sb + k - 2) * kRawRow);
                        if (k == 4) kc[sb][2] = rd_codes(sb, 2);
                        if (k == 5) kc[sb][3] = rd_codes(sb, 3);
                        if (sb == 0 && k == 8) kr[1][0] = rd_rope(1, 0);
                        if (sb == 0 && k == 9) kr[1][1] = rd_rope(1, 1);
                        step(10 * sb + k);
                        if (k < 2) {
                            part[sb][4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[sb][k], qrope[k], part[sb][4], 0, 0, 0);
                        } else {
                            const int u = 2 * ((k - 2) >> 2) + (k & 1);
                            const bool lo = ((k - 2) & 2) != 0;
                            part[sb][u] = mfma_fp8_q(u, kc[sb][u], lo ? qlo[u] : qhi[u], part[sb][u], lo ? qsc_lo : qsc_hi);
                        }
                        // tiles 0, 1 two slots after their last MFMA; tiles 2, 3 of row block
                        // 0 under row block 1's first MFMAs
                        if (k == 7 || k == 8) combine(sb, 0, k - 7);
                        if (sb == 1 && (k == 1 || k == 2)) combine(0, 1, k - 1);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                combine(1, 1, 0);
                combine(1, 1, 1);
            };

            float st_cur[8];                   // S^T of the tile whose softmax is next
            for (int i = 0; ntiles > 0 && i <= ntiles; i++) {
                tile_top(i);                   // tiles i and i + 1 are in LDS
                if (i == ntiles) {
                    break;
                }
                if (i == 0) qk_tile(0, st_cur, [](int) {});
                // ---- softmax of tile i, spread over the MFMA slots of tile i + 1's S^T: logits
                //      and mask, the max over the head's 32 tokens, the lazily moved reference,
                //      p = 2^(s - m) and the row sum; P and the factor for O^T (1 unless the
                //      reference moved) go to the value wave.  (Past the last tile, tile i + 1's
                //      slot holds zeros and its result is unused.)
                uint32_t vmask = 0;
                if (SPARSE) {                      // tokens 8g4 .. 8g4+7: waves 2g4, 2g4+1
                    const uint32_t v2 = *(const uint16_t *)&s_valid[i % kRawSlots][2 * g4];
                    vmask = (v2 & 0xFu) | ((v2 >> 4) & 0xF0u);
                }
                float sv[8], bm = -INFINITY, m_new = m, alpha = 1.f, mref = 0.f, ps = 0.f;
                float pr[8];
                f32x4 scr[8];                      // tile i's token scales, read again
                bf16x8 pb[4];
                auto logits = [&](int r0) {
#pragma unroll
                    for (int r = r0; r < r0 + 4; r++) {
                        const int tok = t0 + kT * i + 8 * g4 + r;
                        const bool vis = SPARSE ? ((vmask >> r) & 1u) != 0
                                                : MASKED ? (tok < tlim && tok >= tlo) : tok < t1;
                        sv[r] = vis ? st_cur[r] * a.scale_log2 : -INFINITY;
                        bm = fmaxf(bm, sv[r]);
                    }
                };
                auto softmax_step = [&](int s) {
                    if (s == 0) logits(0);
                    if (s == 1) logits(4);
                    if (s == 2) {
                        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
                        bm = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
                    }
                    if (s == 3) {
                        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
                        bm = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
                        m_new = bm > m + kLazyMax ? bm : m;
                        alpha = m_new == m ? 1.f : fast_exp2(m - m_new);   // m = -inf: 0
                        mref = m_new == -INFINITY ? 0.f : m_new;
                    }
                    if (s >= 4 && s < 8) {
#pragma unroll
                        for (int r = 2 * (s - 4); r < 2 * (s - 4) + 2; r++) {
                            pr[r] = fast_exp2(sv[r] - mref);
                            ps += pr[r];
                        }
                    }
                    if (s == 8) {
                        l = l * alpha + ps;
                        m = m_new;
                    }
                    // the value waves' B operands: P^T times each value tile's token scales
                    // (the value is the key's first 512 dims, so the scales are the key tile
                    // scales), two rows per slot, from scales read again four slots before
                    if (s >= 5 && s < 9) {
#pragma unroll
                        for (int r = 2 * (s - 5); r < 2 * (s - 5) + 2; r++)
                            scr[r] = *(PA_LDS const f32x4 *)((PA_LDS const uint8_t *)raw[i % kRawSlots] + sc_off + r * kRawRow);
                    }
                    if (s >= 9 && s < 13) {
#pragma unroll
                        for (int r = 2 * (s - 9); r < 2 * (s - 9) + 2; r++) {
#pragma unroll
                            for (int t = 0; t < 4; t++) pb[t][r] = (__bf16)(pr[r] * scr[r][t]);
                        }
                    }
                    if (s == 13) {
                        s_p[i & 1][hg][0][lane] = pb[0];
                        s_p[i & 1][hg][1][lane] = pb[1];
                    }
                    if (s == 14) {
                        s_p[i & 1][hg][2][lane] = pb[2];
                        s_p[i & 1][hg][3][lane] = pb[3];
                        // (the column's 4 lanes hold the same factor: no branch in the body, which
                        // would let the compiler sink the MFMAs and their combines past it)
                        s_alpha[i & 1][hg][col] = alpha;
                    }
                };
                float st_nxt[8];
                qk_tile(i + 1, st_nxt, softmax_step);
#pragma unroll
                for (int r = 0; r < 8; r++) st_cur[r] = st_nxt[r];
            }

            // ---- epilogue: 1 / l (with a sink of a whole-request item) and lse
            l = col_sum(l);
            float inv, lse_v;
            const float sk = (a.sinks && (flags & 1)) ? a.sinks[head0 + col] * 1.4426950408889634f : -INFINITY;
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
            if (g4 == 0) {
                s_inv[hg][col] = inv;
                if (active) {
                    if (flags & 1) a.lse[(int64_t)b * nq * Hq + qr] = lse_v;
                    else if (!SPARSE && a.counters) store_shared(a.ws_lse + (int64_t)it * nq * Hq + qr, lse_v);
                    else a.ws_lse[(int64_t)it * nq * Hq + qr] = lse_v;
                }
            }
            lds_barrier();                                   // s_inv out
        } else {
            // ================= value wave: O^T += V^T P^T of tile i-1 in iteration i, for
            // value tile vt = hg (dims 128 vt .. +127) and all 4 head blocks: O^T block
            // acc[4 d + hb] holds dims 128 vt + 16 d + (4 g4 + e) of head col of block hb, so
            // each V^T operand is read and converted once and feeds 4 MFMAs
            const int vt = hg;
            f32x4 acc[kDvBlocks];
#pragma unroll
            for (int d = 0; d < kDvBlocks; d++) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

            // V^T reads: tile j's dims 128 vt + 16 d + col, tokens 8g4 + 0..7 (lane); the 8
            // reads of the next tile go out before the barrier (the tile is in LDS since the
            // top of this iteration)
            // (the base is made opaque, so that the reads become base + immediate offset and
            // the compiler does not hoist a register per read)
            auto vbase = [&](int t) {
                uint32_t x = lds_addr(raw[t % kRawSlots]) + pv_off + 128 * vt;
                asm volatile("" : "+v"(x));
                return (PA_LDS uint8_t *)(uintptr_t)x;
            };
            auto rd = [&](PA_LDS uint8_t *vb, int d) {
                return __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2 *)(vb + 16 * d));
            };
            i32x2 vw[kVBlocks];
            for (int i = 0; ntiles > 0 && i <= ntiles; i++) {
                tile_top(i);
                if (i > 0) {
                    const int j = i - 1;
                    // the tile's factors for O^T and the B operands (P^T of head block hb
                    // times value tile vt's token scales, from the score wave of hb)
                    float alpha[4];
                    bf16x8 pbt[4];
#pragma unroll
                    for (int hb = 0; hb < 4; hb++) {
                        alpha[hb] = s_alpha[j & 1][hb][col];
                        pbt[hb] = s_p[j & 1][hb][vt][lane];
                    }
                    if (__any(alpha[0] != 1.f || alpha[1] != 1.f || alpha[2] != 1.f || alpha[3] != 1.f)) {
                        mfma_acc_drain(acc);                 // rare: a reference moved
#pragma unroll
                        for (int d = 0; d < kDvBlocks; d++) acc[d] = acc[d] * alpha[d & 3];
                        mfma_acc_drain(acc);                 // (wait states before the MFMAs)
                    }
                    // A = V^T converted to bf16 two blocks ahead; the first two get their wait
                    // states before the first MFMA explicitly (the asm MFMAs are invisible to
                    // the compiler's hazard checks)
                    bf16x8 va[3];
                    va[0] = fp8x8_to_bf16((uint32_t)vw[0][0], (uint32_t)vw[0][1]);
                    va[1] = fp8x8_to_bf16((uint32_t)vw[1][0], (uint32_t)vw[1][1]);
                    asm volatile("s_nop 1" : "+v"(va[0]), "+v"(va[1]));
#pragma unroll
                    for (int d = 0; d < kVBlocks; d++) {
#pragma unroll
                        for (int hb = 0; hb < 4; hb++) mfma_acc(acc[4 * d + hb], va[d % 3], pbt[hb]);
                        if (d + 2 < kVBlocks)
                            va[(d + 2) % 3] = fp8x8_to_bf16((uint32_t)vw[d + 2][0], (uint32_t)vw[d + 2][1]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if (i < ntiles) {
                    PA_LDS uint8_t *vbn = vbase(i);
#pragma unroll
                    for (int d = 0; d < kVBlocks; d++) vw[d] = rd(vbn, d);
                }
            }
            mfma_acc_drain(acc);
            lds_barrier();                                   // s_inv in
            // ---- epilogue: rows of head block hb: draft token and heads as in the score wave
#pragma unroll
            for (int hb = 0; hb < 4; hb++) {
                const int r0 = group * kHeadsPerWG + hb * kHeadsPerWave;
                if (r0 >= G * nq) continue;                  // no query rows
                const int q_i = r0 / G;
                const int64_t row = (int64_t)q_i * Hq + (r0 - q_i * G) + col;
                const float inv = s_inv[hb][col];
                if (flags & 1) {
                    uint16_t *orow = a.out + ((int64_t)b * nq * Hq + row) * kDv + 128 * vt + 4 * g4;
#pragma unroll
                    for (int d = 0; d < kVBlocks; d++) {
                        bf16x4 o;
#pragma unroll
                        for (int e = 0; e < 4; e++) o[e] = (__bf16)(acc[4 * d + hb][e] * inv);
                        *(bf16x4 *)(orow + 16 * d) = o;
                    }
                } else {
                    float *orow = a.ws_o + ((int64_t)it * nq * Hq + row) * kDv + 128 * vt + 4 * g4;
                    if (!SPARSE && a.counters) {         // merged inside this launch
#pragma unroll
                        for (int d = 0; d < kVBlocks; d++) {
#pragma unroll
                            for (int e = 0; e < 4; e++) store_shared(orow + 16 * d + e, acc[4 * d + hb][e] * inv);
                        }
                    } else {
#pragma unroll
                        for (int d = 0; d < kVBlocks; d++) *(f32x4 *)(orow + 16 * d) = acc[4 * d + hb] * inv;
                    }
                }
            }
        }
        wait_vmcnt<0>();
        lds_barrier();                                       // the item's LDS is free
    }
    // fused combine (dense, one query token: the head group is heads [64 group, 64 group +
    // 64)): the last workgroup to finish a request's chunks merges them
    if (!SPARSE && a.counters)
        fused_combine_tail(a, plan, part, ib, ie, group, ngroups, group * kHeadsPerWG,
                           min(kHeadsPerWG, G - group * kHeadsPerWG), 1, &s_flag);
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
