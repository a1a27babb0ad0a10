// Split-KV MQA decode over the MLA 656-byte FP8 latent cache (D_qk = 576, D_v = 512,
// one KV head shared by G query heads, G a multiple of 16 up to 128), gfx950.
//
// Token layout (FlashMLA walk-through, section 数据加载, byte-layout table): 512 e4m3
// codes, 4 fp32 scales (one per 128 codes), 64 bf16 rope values.  The key is the 576
// dequantised values, the value is their first 512 (V shares the latent with K).  Both
// products run as bf16 MFMAs with fp32 accumulation, as the walk-through's kernel does
// (same section): the codes are converted to bf16 exactly (every e4m3 value is a bf16
// value) and the per-token tile scales are applied in fp32, to the score partials of each
// 128-dim tile and to the probabilities of each 128-dim value tile.
//
// One workgroup (12 waves, three per SIMD) = one (part, group of 64 query rows); it walks
// the part's items.  Query rows are (draft token qi, head g) pairs, row qi * G + g, so with
// several query tokens per request (a linear speculative draft) each block of 16 rows
// shares one draft token and its causal limit L - q_len + qi + 1.  The two head groups of a
// part run as workgroups 8 ids apart, i.e. on the same XCD at about the same time, so the
// second read of each KV tile is an L2 hit (the FlashMLA walk-through shares one KV tile
// between two 64-head CTAs through a cluster, section 计算环节一; here the L2 of the XCD
// plays that role).
//
// Waves hg, hg + 4 and hg + 8 share a SIMD (the FlashMLA walk-through splits a tile's work
// over two warpgroups, section 计算环节二; here the split is by operation and by tokens):
//   * score waves (hg, sb), sb = 0, 1: Q of head block hg resident (bf16, 72 registers);
//     wave sb computes S^T = K . Q^T for the 16 tokens of row block sb of each 32-token
//     tile, in iteration i the MFMAs of tile i+1 with tile i's softmax between them.  The
//     two halves of a tile agree on one running maximum: each publishes its half's
//     per-head maximum through LDS one iteration ahead, and both move the reference
//     identically; each keeps its own partial row sum, added at the end of the item;
//   * value wave hg (O^T of value dims 128 hg .. +127 for all 64 heads resident, 128
//     registers) runs O^T += V^T . P^T of tile i-1 in iteration i: each V^T operand is read
//     and converted once and feeds the 4 head blocks' MFMAs.
// A wave issues VALU work at about one instruction per 6 cycles, while a SIMD completes
// one every 2.5-4.5 cycles when two or more waves issue: splitting a tile's score work
// (code conversions, tile-scale combination, softmax) over two waves per head block puts
// two VALU streams beside the value wave's matrix stream on each SIMD.
//
// Per 32-token tile:
//   * the tokens' 656 bytes go HBM -> LDS by direct-to-LDS loads (one instruction per
//     token, 41 lanes of 16 bytes; a token that is not real reads as zeros) into a 5-slot
//     ring of 21,856-byte tile slots (token rows placed for conflict-free reads, raw_row);
//     each value wave loads 8 tokens, tile i+3's one per 16-dim block of its PV MFMAs in
//     iteration i (tiles i and i+1 are waited for at its top: the score waves read tile
//     i+1's keys).  Page ids come the same way, 3 tiles ahead, into a small LDS ring (a
//     scalar load would make every later LDS wait also wait for it);
//   * scores: rope dims: two bf16 MFMAs 16x16x32 (first, so that their partial starts the
//     sum); per 128-dim scale tile u, four on the codes converted in registers;
//     S = q_rope . k_rope + sum_u scale_t,u (q_u . code_t,u) in fp32; the logit scale c > 0
//     joins in the maximum and in the exponent, p = 2^(c S - m);
//   * an online softmax per head column (the previous tile's, in the MFMA slots of the next
//     tile's scores); the score waves write P^T times each 128-dim value tile's token
//     scales (bf16, the B operands of the PV MFMAs; each wave its half of the tokens) and
//     the factor for O^T (1 unless the reference max moved);
//   * O^T += V^T . P^T with bf16 MFMA 16x16x32, V^T read transposed from the FP8 codes
//     (ds_read_b64_tr_b8) and converted in registers (exact).  O^T takes 128 registers (the
//     register-budget problem the FlashMLA walk-through describes in section 计算环节二),
//     ordinary VGPRs.
// Operand layouts.  QK row block sb of the A operand holds, in MFMA row m = 4g + r, token
// 8g + 4sb + r, so lane group g of the S^T result holds tokens 8g + 4sb + 0..3: the k slots
// 4sb .. 4sb+3 of lane group g of the PV B operand (B = P^T, k = 8g + j), and the
// transposed read returns tokens 8g..8g+7 of one value dim per lane; the PV operands pass
// through LDS lane for lane, each score wave writing its 8 bytes of the 16.  In a QK MFMA,
// lane (col, g) holds dims 16g + 0..7, 16g + 8..15, 64 + 16g + 0..7, 64 + 16g + 8..15 of
// the 128-dim tile (one per k-step), the same for K and Q.
// One workgroup barrier per tile: it publishes the PV operands and half-tile maxima, and
// frees the ring slot of tile i-2.  The running max is only moved when a tile's max
// exceeds it by more than 8 (log2 units), so the rescale of O^T is rare; probabilities stay
// below 2^8 and the result is the same up to rounding (the reference cancels in the final
// normalisation).
//
// Sparse decode (FlashMLA walk-through, section 调度: the decode call takes sparse
// indices): the items then cover index slots, and slot k of request b names the key
// position indices[b][k].  The address of a listed token takes two dependent lookups
// (index, then block table); lanes 0-7 of each value wave (its 8 tokens of a tile) load
// them direct to LDS, positions 6 tiles and page ids 3 tiles ahead of the tile's own
// loads, so that every wait for them is one the KV ring does anyway; the 8 token addresses
// are then worked out on the vector unit, one lane per token.  A slot outside the item or
// the request loads nothing (zeros), and a per-tile bit mask of the real tokens is
// applied in the softmax.
#include "pa_internal.h"
#include "pa_merge.h"

#include <cfloat>
#include <utility>

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
struct u32x4x2 {
    u32x4 x, y;
};

#define PA_LDS __attribute__((address_space(3)))

constexpr int kScoreWaves = 8;                     // head block hg = w & 3, row block sb = w >> 2
constexpr int kValueWaves = 4;                     // value tile vt = w & 3
constexpr int kWaves = kScoreWaves + kValueWaves;  // three per SIMD: waves w, w + 4, w + 8
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = 4 * kHeadsPerWave;     // 64
constexpr int kDqk = 576, kDv = 512;
constexpr int kTokBytes = 656;
constexpr int kChunks = kTokBytes / 16;            // 41 16-byte chunks per token
constexpr int kT = 32;                             // tokens per tile
constexpr int kLoadWaves = kValueWaves;           // the value waves issue the tile loads
constexpr int kTokPerWave = kT / kLoadWaves;       // 8 tokens loaded per value wave and tile
// LDS placement of a tile's 32 token rows (see raw_row): groups of 4 consecutive tokens,
// rows 672 bytes apart inside a group; group j starts at kGroupQuad[j] 16-byte units
constexpr int kRowStep = 672;                      // bytes between the rows of a group
constexpr int kGroupQuad[8] = {0, 167, 344, 511, 688, 855, 1032, 1199};
constexpr int kHalfGroupBytes = 167 * 16;          // from token 0 to token 4 of a wave's 8
constexpr int kRawTile = (1199 + 3 * 42 + 41) * 16;   // 21856: the last row's end
constexpr int kRawSlots = 5;                       // tile ring
constexpr int kAhead = kRawSlots - 2;              // loads go out 3 tiles ahead (2 ahead of the keys'
                                                   // first use); lookups: page ids 3 (sparse:
                                                   // positions 6) tiles ahead
constexpr int kLookRing = 8;                       // lookup slots (tiles) per wave
constexpr int kDvBlocks = kDv / 16;                // O^T blocks of a value wave (8 dims x 4 heads), 32 MFMAs a tile
constexpr int kVBlocks = 128 / 16;                 // 16-dim blocks of a value wave's value tile
constexpr float kLazyMax = 8.0f;                   // log2 units

static_assert(kRawSlots >= 4, "the tile loop reads tiles i and i-1 with loads in flight");
static_assert(kTokPerWave == 128 / 16, "a value wave issues one token load per 16-dim block of its PV");
static_assert(kLookRing > 2 * kAhead && (kLookRing & (kLookRing - 1)) == 0, "lookup ring");

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}) in order
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// LDS byte offset of token row r (0..31) in a tile slot.  LDS has 64 four-byte banks; a
// 16-byte read serves 16 lanes per cycle, lanes {0-3, 12-15, 20-23, 24-27} together and
// {4-11, 16-19, 28-31} together (then the same for lanes 32-63), an 8-byte read lanes 0-31,
// then 32-63 (both measured on MI355X, lane pair by lane pair).  A score wave's operand read
// takes, in lane quad 4 g4 + c, the rows of group 2c + sb at column 16 g4; the transposed
// value read takes rows 8 g4 + 0..7.  With group j's 4 rows 42 16-byte units apart (bank
// groups p_j + {0, 10, 4, 14} mod 16), both are conflict-free when the group starts sit at
// bank groups p0 = p4 = 0, p2 = p6 = 8 (row block 0) and p1 = p5 = 7, p3 = p7 = 15 (row
// block 1): each cycle's 16 rows then cover all 16 bank groups (counted with
// SQ_LDS_BANK_CONFLICT on MI355X: 0 for both reads, where 752-byte rows had a 2-way
// conflict on the operand reads).  The groups are packed into 21,856 bytes.
__device__ __forceinline__ int raw_row(int r)
{
    const int k = r >> 3;                          // pair of groups (2k, 2k + 1)
    return (k == 0 ? 0 : k == 1 ? 344 * 16 : k == 2 ? 688 * 16 : 1032 * 16) + ((r >> 2) & 1) * kHalfGroupBytes +
           (r & 3) * kRowStep;
}
static_assert(kGroupQuad[1] - kGroupQuad[0] == 167 && kGroupQuad[3] - kGroupQuad[2] == 167 &&
              kGroupQuad[5] - kGroupQuad[4] == 167 && kGroupQuad[7] - kGroupQuad[6] == 167 &&
              kGroupQuad[2] == 344 && kGroupQuad[4] == 688 && kGroupQuad[6] == 1032,
              "raw_row and the loads place the second 4 tokens of each 8 at a fixed distance");
static_assert(kGroupQuad[7] * 16 + 3 * kRowStep + kTokBytes <= kRawTile, "last row inside the slot");
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool SPARSE>
struct MlaCfg {
    // loads per value wave and tile: one per token, one page-id load (sparse: plus one index
    // load)
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
// a + b * c in 64 bits on the scalar unit, for uniform operands (b < 2^31).  The compiler
// selects a vector multiply-add for 64-bit products even of uniform values; a vector
// 64-bit multiply-add costs four times a plain vector instruction and its result then
// needs moving back to scalar registers.
__device__ __forceinline__ uint64_t s_mad64(uint64_t a, uint32_t b, uint64_t c)
{
    uint32_t lo, hi, t;
    asm("s_mul_i32 %0, %3, %4\n\t"
        "s_mul_hi_u32 %1, %3, %4\n\t"
        "s_mul_i32 %2, %3, %5\n\t"
        "s_add_i32 %1, %1, %2\n\t"
        "s_add_u32 %0, %0, %6\n\t"
        "s_addc_u32 %1, %1, %7"
        : "=&s"(lo), "=&s"(hi), "=&s"(t)
        : "s"(b), "s"((uint32_t)c), "s"((uint32_t)(c >> 32)), "s"((uint32_t)a), "s"((uint32_t)(a >> 32))
        : "scc");
    return ((uint64_t)hi << 32) | lo;
}
// (the row base in scalar registers, the lane's byte offset in a vector register: no 64-bit
// vector address is kept across the tile loop; the offsets stay below 2^28, since a request
// has at most 2^26 pages and 2^24 indices)
__device__ __forceinline__ void lds_dma_glb4(const void *row, uint32_t byte_off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(byte_off), "s"(row) : "memory", "m0");
}
// a row pointer that is the same in every lane, in scalar registers
template <typename T>
__device__ __forceinline__ const T *uniform_ptr(const T *p)
{
    const uint64_t x = (uint64_t)p;
    return (const T *)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x));
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

// max(a, b) as one instruction: fmaxf quiets signalling NaN inputs first, which costs an
// instruction per operand the compiler cannot prove canonical (values from LDS or from
// lane permutes).  The operands here are logits or -inf, never NaN.
__device__ __forceinline__ float max_nc(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// max / sum over the lanes l, l^16, l^32, l^48 (the 4 row groups of one MFMA column),
// through the row-swap permutes (no LDS); the result is the same in all four lanes
__device__ __forceinline__ float col_max(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max_nc(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max_nc(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float col_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
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
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void pa_mla_kernel(
    DecodeArgs a, const int32_t *__restrict__ plan, const int32_t *__restrict__ bt, int ngroups,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ indices)
{
    constexpr int kLoadsPerTile = MlaCfg<SPARSE>::kLoadsPerTile;
    __shared__ __attribute__((aligned(16))) uint8_t raw[kRawSlots][kRawTile];
    // the PV B operands of a tile from the score waves of head block hg, in their lanes'
    // layout (lane (col, g4): head col, tokens 8g4 + 0..7, of which row block sb holds
    // 8g4 + 4sb + 0..3): P^T times value tile t's token scales, bf16, [tile parity][hg]
    // [value tile t][sb][lane]; each score wave writes 512 contiguous bytes (a half-slot
    // write per lane, 16 bytes apart, would meet the same banks four times)
    __shared__ bf16x4 s_p[2][4][4][2][64];
    __shared__ float s_alpha[2][4][16];       // factor on O^T before the tile's PV, per head
    __shared__ float s_tmax[2][2][4][16];     // [tile parity][sb][hg][head]: half-tile maxima
    __shared__ float s_lsum[2][4][16];        // [sb][hg][head]: the halves' row sums
    __shared__ float s_inv[4][16];            // the item's final 1 / l, per head
    __shared__ int s_flag;                    // fused combine: this workgroup merges
    __shared__ __attribute__((aligned(4))) uint8_t s_valid[kRawSlots][kLoadWaves];   // sparse: real-token bits
    // lookups: [position | page id][tile % kLookRing][load wave][token] (dense: page ids of
    // the wave's first token only)
    __shared__ int32_t s_look[2 * kLookRing * kLoadWaves * kTokPerWave];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int hg = wave & 3;                       // score: head block; value: value tile (same SIMD)
    const bool scorer = wave < kScoreWaves;        // score wave; else value wave
    const int sb = (wave >> 2) & 1;                // score wave: row block of each tile
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

    // LDS byte offsets inside a tile slot: the QK operand rows of this wave's row block
    // (token 8(col/4) + 4 sb + col%4 at this lane's 16 bytes of each 64-dim group), the
    // rope operand, the scale rows of this lane's tokens 8g4 + 4sb + r, and the transposed
    // PV read (lane pair 2r, 2r+1 of a 16-lane block supplies row 8g4 + r, bytes 0-7 and
    // 8-15 of the block's 16 value dims)
    // (the scale rows 8g4 + 4sb + 0..3 are one group of 4, kRowStep apart)
    const uint32_t qk_off = (uint32_t)(raw_row(8 * (col >> 2) + 4 * sb + (col & 3)) + 16 * g4);
    const uint32_t rope_off = qk_off + 528;
    const uint32_t sc_off = (uint32_t)(raw_row(8 * g4 + 4 * sb) + 512);
    const uint32_t pv_off = (uint32_t)(raw_row(8 * g4 + ((lane & 15) >> 1)) + 8 * (lane & 1));

    // a fixed-split plan has exactly one item per part (no plan read on the critical path)
    const int ib = a.fixed_splits > 0 ? part : plan[a.part_begin_off + part];
    const int ie = a.fixed_splits > 0 ? part + 1 : plan[a.part_begin_off + part + 1];

    // The two roles run the same items with the same barrier sequence, each in its own
    // loop (values one role keeps across its items then never occupy the other's registers).
    if (scorer) {
        // issue priority on the SIMD (oldest wave first by default): value wave, then score
        // half 1, then score half 0; measured -5 % kernel time on the MLA workload
        if (sb) __builtin_amdgcn_s_setprio(1);
        for (int it = ib; it < ie; it++) {
            const int b = plan[a.items_off + 4 * it + 0];
            const int t0 = plan[a.items_off + 4 * it + 1];
            const int t1 = plan[a.items_off + 4 * it + 2];
            const int flags = plan[a.items_off + 4 * it + 3];
            const int ntiles = (t1 - t0 + kT - 1) / kT;
            const int64_t qr = (int64_t)qi * Hq + head0 + col;     // query row within the request

            // ---- the value waves load the tiles; top of tile i: all waves are past tile i-1
            //      and tiles i and i + 1 are in LDS
            auto tile_top = [&](int) { lds_barrier(); };
            if (ntiles > 0) lds_barrier();                   // tile 0 is in

                // ================= score wave (hg, sb): S, softmax and P of row block sb of tile i
                // causal limit of the block's draft token and the first key its window leaves
                int tlim = t1, tlo = 0;
                if (MASKED) {
                    const int L = seq_lens[b];
                    if (nq > 1) tlim = min(t1, L - (nq - 1 - qi));
                    if (a.window > 0) tlo = max(0, L - nq + qi - a.window + 1);
                }
                // Q^T of the block's 16 heads (B of the MFMAs), resident, bf16.  Latent tile u,
                // k-step e: lane (col, g4) holds dims 128u + 64(e >> 1) + 16g4 + 8(e & 1) .. +7.
                // Rope: step r <- dims 512 + 32r + 8g4 .. +7.  A block with no query rows runs on
                // a zero Q and writes nothing.
                bf16x8 qb[4][4], qrope[2];
                {
                    const uint16_t *qrow = a.q + ((int64_t)b * nq * Hq + qr) * kDqk;
#pragma unroll
                    for (int u = 0; u < 4; u++) {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            qb[u][e] = active ? *(const bf16x8 *)(qrow + 128 * u + 64 * (e >> 1) + 16 * g4 + 8 * (e & 1))
                                              : bf16x8{};
                    }
#pragma unroll
                    for (int r = 0; r < 2; r++)
                        qrope[r] = active ? *(const bf16x8 *)(qrow + 512 + 32 * r + 8 * g4) : bf16x8{};
                }
                // reference max (log2 domain) of head `col`, both halves; starts at the lowest
                // finite value, so that the reference and the factor need no -inf case
                float m = -FLT_MAX;
                float l = 0.f;           // this lane's share of the row sum (its 4 tokens)

                // ---- S^T of row block sb of tile t (rows: this lane's tokens 8g4 + 4sb + r) into
                //      st[4]: per 128-dim scale tile u an fp32 partial of 4 bf16 MFMAs on the
                //      converted codes, one partial for the rope dims (2 bf16 MFMAs), combined
                //      with the token scales in fp32 as the tiles complete.  MFMA slots 0, 1: rope;
                //      slot k >= 2: tile (k - 2) / 4, step (k - 2) % 4; the A operand of a slot is
                //      converted in the slot before, codes are read 3 slots before that.
                //      step(k) runs in slot k, before its MFMA: the VALU work of the previous
                //      tile, issued while the matrix core works.
                // the token scales of the tile whose S^T was computed last (token 8g4 + 4sb + r,
                // tiles u = 0..3): written by qk_tile, used by its tile's combine and, one
                // iteration later, by that tile's P^T scaling
                f32x4 sc4[4];
                auto qk_tile = [&](int t_slot, float (&st)[4], auto &&step) {
                    PA_LDS const uint8_t *slot = (PA_LDS const uint8_t *)raw[t_slot];
                    auto rd_codes = [&](int u) {
                        PA_LDS const uint8_t *p = slot + qk_off + 128 * u;
                        const u32x4 x = *(PA_LDS const u32x4 *)p;
                        const u32x4 y = *(PA_LDS const u32x4 *)(p + 64);
                        return u32x4x2{x, y};
                    };
                    auto cvt = [&](const u32x4x2 &c, int e) {
                        const u32x4 &w = (e >> 1) ? c.y : c.x;
                        return (e & 1) ? fp8x8_to_bf16(w[2], w[3]) : fp8x8_to_bf16(w[0], w[1]);
                    };
                    u32x4x2 kc[2];                     // codes of tiles u (kc[u & 1])
                    bf16x8 kr[2];
                    f32x4 part[5];
                    float x[4];
#pragma unroll
                    for (int p = 0; p < 5; p++) part[p] = f32x4{0.f, 0.f, 0.f, 0.f};
                    kr[0] = *(PA_LDS const bf16x8 *)(slot + rope_off);
                    kr[1] = *(PA_LDS const bf16x8 *)(slot + rope_off + 64);
                    kc[0] = rd_codes(0);
                    bf16x8 av[2];
#pragma unroll
                    for (int k = 0; k < 18; k++) {
                        const int j = k - 2;           // latent step of slot k >= 2
                        // reads issued at this slot: the next tile's codes 3 slots before their
                        // conversion; the 4 tiles' scales of each token (one 16-byte row) once
                        // the previous tile's P^T scaling (steps 4 - 7) is done with sc4
                        if (j >= 0 && (j & 3) == 0 && j + 4 < 16) kc[((j >> 2) + 1) & 1] = rd_codes((j >> 2) + 1);
                        if (k == 8) {
#pragma unroll
                            for (int r = 0; r < 4; r++) sc4[r] = *(PA_LDS const f32x4 *)(slot + sc_off + r * kRowStep);
                        }
                        step(k);
                        if (k < 2) {
                            part[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[k], qrope[k], part[4], 0, 0, 0);
                        } else {
                            part[j >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j & 1], qb[j >> 2][j & 3], part[j >> 2], 0, 0, 0);
                        }
                        if (k >= 1 && j + 1 < 16) av[(j + 1) & 1] = cvt(kc[((j + 1) >> 2) & 1], (j + 1) & 3);
                        // the token scales times the tile partials: tile 0's five slots after
                        // its last MFMA (two after its scales are read), tiles 1 and 2 three
                        // slots after, tile 3's after the loop; the rope partial starts the sum
                        if (k == 10 || k == 12 || k == 16) {
                            const int u = k == 10 ? 0 : (k - 8) >> 2;
#pragma unroll
                            for (int r = 0; r < 4; r++) {
                                float y = u == 0 ? part[4][r] : x[r];
                                y += sc4[r][u] * part[u][r];
                                asm volatile("" : "+v"(y));    // computed in this slot
                                x[r] = y;
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; r++) st[r] = x[r] + sc4[r][3] * part[3][r];
                };

                // ---- logits of row block sb of tile t (log2 domain, masked) and their max per
                //      head, published for the other half of the tile
                float sv[4], bm_own = -INFINITY;
                auto finish_tile = [&](int t, int t_slot, int t_par, const float (&st)[4]) {
                    uint32_t vmask = 0;
                    if (SPARSE)                        // tokens 8g4 + 4sb + r: loader g4, bits 4sb + r
                        vmask = (uint32_t)s_valid[t_slot][g4] >> (4 * sb);
                    float mx = -INFINITY;
                    if (!SPARSE && !MASKED && t0 + kT * (t + 1) <= t1) {
                        // a tile wholly inside the item (all but the last): no mask (a uniform
                        // branch; the mask costs ~12 vector instructions per tile)
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            sv[r] = st[r];
                            mx = fmaxf(mx, sv[r]);
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const int tok = t0 + kT * t + 8 * g4 + 4 * sb + r;
                            const bool vis = SPARSE ? ((vmask >> r) & 1u) != 0
                                                    : MASKED ? (tok < tlim && tok >= tlo) : tok < t1;
                            sv[r] = vis ? st[r] : -INFINITY;    // unscaled; the scale c > 0 joins in
                            mx = fmaxf(mx, sv[r]);                //   the max and the exponent
                        }
                    }
                    bm_own = col_max(mx) * a.scale_log2;
                    if (g4 == 0) s_tmax[t_par][sb][hg][col] = bm_own;
                };

                {
                    float st0[4];
                    if (ntiles > 0) {
                        qk_tile(0, st0, [](int) {});
                        finish_tile(0, 0, 0, st0);
                    }
                }
                // one iteration: softmax of tile i, S^T of tile i + 1.  The ring slots and the
                // parity are compile-time constants of the unrolled loop below (LDS offsets
                // become immediates instead of a vector add per address and tile).
                auto iteration = [&](int i, auto SLOT_I, auto SLOT_N, auto PAR) {
                    constexpr int slot_i = decltype(SLOT_I)::value, slot_n = decltype(SLOT_N)::value;
                    constexpr int par = decltype(PAR)::value;
                    // ---- softmax of tile i, spread over the MFMA slots of tile i + 1's S^T: the
                    //      tile's max (both halves), the lazily moved reference, p = 2^(s - m) and
                    //      this lane's row sum; P and the factor for O^T (1 unless the reference
                    //      moved) go to the value wave.  (Past the last tile, tile i + 1's slot
                    //      holds zeros and its result is unused.)
                    float bm_other = 0.f, m_new = m, alpha = 1.f, mref = 0.f, ps = 0.f;
                    float pr[4];
                    bf16x4 pb[4];
                    auto softmax_step = [&](int s) {
                        if (s == 0) bm_other = s_tmax[par][sb ^ 1][hg][col];
                        if (s == 2) {
                            const float bm = max_nc(bm_own, bm_other);
                            m_new = bm > m + kLazyMax ? bm : m;
                            alpha = fast_exp2(m - m_new);      // exactly 1 if unmoved, 0 from the start
                            mref = m_new;
                        }
                        if (s == 3 || s == 4) {
#pragma unroll
                            for (int r = 2 * (s - 3); r < 2 * (s - 3) + 2; r++) pr[r] = fast_exp2(fmaf(sv[r], a.scale_log2, -mref));
                            ps = s == 3 ? pr[0] + pr[1] : ps + (pr[2] + pr[3]);
                        }
                        if (s == 5) {
                            l = l * alpha + ps;
                            m = m_new;
                        }
                        // the value waves' B operands: P^T times each value tile's token scales
                        // (the value is the key's first 512 dims, so the scales are the key tile
                        // scales, kept in sc4 from tile i's S^T)
                        if (s >= 4 && s < 8) {
                            const int r = s - 4;
#pragma unroll
                            for (int t = 0; t < 4; t++) pb[t][r] = (__bf16)(pr[r] * sc4[r][t]);
                        }
                        if (s == 11 || s == 12) {
#pragma unroll
                            for (int t = 2 * (s - 11); t < 2 * (s - 11) + 2; t++)
                                s_p[par][hg][t][sb][lane] = pb[t];
                        }
                        if (s == 13) {
                            // both halves hold the same factor and both write it (no branch in the
                            // body, which would let the compiler sink the MFMAs past it)
                            s_alpha[par][hg][col] = alpha;
                        }
                    };
                    float st_nxt[4];
                    qk_tile(slot_n, st_nxt, softmax_step);
                    finish_tile(i + 1, slot_n, par ^ 1, st_nxt);
                };
                // iterations i = 0 .. ntiles (the last only meets the barrier), unrolled by 10
                // (the ring's 5 slots x the 2 parities)
                static_assert(10 % kRawSlots == 0, "the unrolled loop cycles through the ring's slots");
                bool done = ntiles <= 0;
                for (int i0 = 0; !done; i0 += 10) {
                    static_for<10>([&](auto U) {
                        constexpr int u = decltype(U)::value;
                        if (done) return;
                        const int i = i0 + u;
                        tile_top(i);           // tiles i and i + 1 are in LDS, tile i's maxima out
                        if (i == ntiles) {
                            done = true;
                            return;
                        }
                        iteration(i, std::integral_constant<int, u % kRawSlots>{},
                                  std::integral_constant<int, (u + 1) % kRawSlots>{}, std::integral_constant<int, u & 1>{});
                    });
                }

                // ---- epilogue: the row sum of both halves, 1 / l (with a sink of a whole-request
                //      item) and lse
                l = col_sum(l);
                if (g4 == 0) s_lsum[sb][hg][col] = l;
                lds_barrier();                                   // both halves' sums out
                if (sb == 0) {
                    l = s_lsum[0][hg][col] + s_lsum[1][hg][col];
                    float inv, lse_v;
                    const float sk = (a.sinks && (flags & 1)) ? a.sinks[head0 + col] * 1.4426950408889634f : -INFINITY;
                    const float M2 = fmaxf(m, sk);
                    if (M2 == -INFINITY || (sk == -INFINITY && l == 0.f)) {
                        inv = 0.f;                               // nothing to attend to
                        lse_v = -INFINITY;
                    } else {
                        // a sink (whole-request items only; split requests get it in the merge)
                        // joins the denominator: den = l 2^(m - M2) + 2^(sk - M2)
                        const float fm = fast_exp2(m - M2);      // m = -inf: 0
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
                }
                lds_barrier();                                   // s_inv out
            wait_vmcnt<0>();
            lds_barrier();                                   // the item's LDS is free
        }
    } else {
        // the value wave issues first on its SIMD (its 32 MFMAs and the tile loads are the
        // longest chain of the three), then the later score half
        __builtin_amdgcn_s_setprio(2);
        for (int it = ib; it < ie; it++) {
            const int b = plan[a.items_off + 4 * it + 0];
            const int t0 = plan[a.items_off + 4 * it + 1];
            const int t1 = plan[a.items_off + 4 * it + 2];
            const int flags = plan[a.items_off + 4 * it + 3];
            const int ntiles = (t1 - t0 + kT - 1) / kT;

            const int lw = wave - kScoreWaves;               // loader index
            // ---- lookups.  Sparse: lane l < 8 loads those of token l of the wave's 8 in tile
            //      j, index slot k.  Dense: lane 0 loads the page id of the wave's first token of
            //      tile j (its 8 tokens are consecutive slots of one page: tiles start at
            //      multiples of 32 tokens and pages hold a multiple of 16).
            const int Lb = SPARSE ? seq_lens[b] : 0;
            auto sp_slot = [&](int j) { return t0 + kT * j + kTokPerWave * lw + (lane & (kTokPerWave - 1)); };
            auto look = [&](int which, int j) {
                return &s_look[((which * kLookRing + (j & (kLookRing - 1))) * kLoadWaves + lw) * kTokPerWave];
            };
            const int32_t *bt_row = uniform_ptr(bt + (int64_t)b * a.max_pages);
            const int32_t *ix_row = SPARSE ? uniform_ptr(indices + (int64_t)b * a.topk) : nullptr;
            auto sp_issue_pos = [&](int j) {           // slots past the row: its last entry
                if (lane < kTokPerWave)
                    lds_dma_glb4(ix_row, 4u * (uint32_t)min(sp_slot(j), a.topk - 1), lds_addr(look(0, j)));
            };
            auto sp_issue_page = [&](int j, int pos) { // no real token: the row's first page
                const bool ok = sp_slot(j) < t1 && pos >= 0 && pos < Lb;
                if (lane < kTokPerWave)
                    lds_dma_glb4(bt_row, 4u * (uint32_t)(ok ? pos >> a.page_shift : 0), lds_addr(look(1, j)));
            };
            auto sp_read = [&](int which, int j) {     // a lookup that is in; lane l: token l % 4
                int v;
                asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v)
                             : "v"(lds_addr(look(which, j)) + 4 * (lane & (kTokPerWave - 1))) : "memory");
                return v;
            };
            auto dn_issue_page = [&](int j) {          // past the item: its last token's page
                if (lane == 0)
                    lds_dma_glb4(bt_row, 4u * (uint32_t)(min(t0 + kT * j + kTokPerWave * lw, t1 - 1) >> a.page_shift),
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

            // ---- loads of tile t into its ring slot: token tt of value wave lw (tile row
            //      8 lw + tt) by lanes 0-40 through a buffer over that token's 656 bytes,
            //      or over none (reads as zeros) when it is not real.  prep_tile works out
            //      where the tokens are (sparse: the page ids of tile t + kAhead and the
            //      positions of tile t + 2 kAhead go out first; the lookups this uses were
            //      loaded kAhead tiles ago), dma_token issues one token's load, end_tile the
            //      tile's last load (dense: the page id of tile t + kAhead).  The value waves
            //      issue a tile's 8 token loads one per 16-dim block of their PV MFMAs: a
            //      burst of all of them at the loop top stalls the issue for hundreds of cycles.
            struct TileLoads {
                const uint8_t *tok;                // dense: the first token's bytes (uniform)
                int nreal;                         // dense: real tokens of the 8; sparse: their bits
                uint64_t toff[kTokPerWave];        // sparse: byte offsets of the 8 tokens in the pool (uniform)
                uint32_t lds0;                     // LDS row of the first token
            };
            auto prep_tile = [&](int t, int page) {
                TileLoads L;
                L.lds0 = (uint32_t)uniform((int)lds_addr(&raw[t % kRawSlots][raw_row(kTokPerWave * lw)]));
                L.tok = nullptr;
                L.nreal = 0;
#pragma unroll
                for (int tt = 0; tt < kTokPerWave; tt++) L.toff[tt] = 0;
                if (SPARSE) {
                    const int pos_look = sp_read(0, t + kAhead);
                    sp_issue_page(t + kAhead, pos_look);
                    sp_issue_pos(t + 2 * kAhead);
                    // lane l works out token l % 8 of the wave's 8 (all 8 at once on the vector
                    // unit; per token on the scalar unit this took ~40 instructions)
                    const int pos = sp_read(0, t);
                    const int pgv = sp_read(1, t);
                    const int k = t0 + kT * t + kTokPerWave * lw + (lane & (kTokPerWave - 1));
                    const bool vis = k < t1 && pos >= 0 && pos < Lb;
                    const uint64_t off = vis ? (uint64_t)(uint32_t)pgv * (uint64_t)a.s_page_b +
                                                   (uint64_t)((uint32_t)(pos & page_mask) * (uint32_t)a.s_tok_b)
                                             : 0;
#pragma unroll
                    for (int tt = 0; tt < kTokPerWave; tt++)
                        L.toff[tt] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(off >> 32), tt) << 32) |
                                     (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)off, tt);
                    const uint32_t vm = (uint32_t)__ballot(vis) & ((1u << kTokPerWave) - 1);
                    L.nreal = (int)vm;             // sparse: the real-token bits
                    if (lane == 0) s_valid[t % kRawSlots][lw] = (uint8_t)vm;
                } else {
                    // the 8 tokens are consecutive slots of one page; addresses on the scalar
                    // unit (the token stride is below 2^20 bytes)
                    const int tw = uniform(t0 + kT * t + kTokPerWave * lw);   // first of the 8 tokens
                    const uint64_t pg = s_mad64((uint64_t)(uintptr_t)a.k_pool, (uint32_t)page, (uint64_t)a.s_page_b);
                    L.tok = (const uint8_t *)(uintptr_t)(pg + (uint32_t)(tw & page_mask) * (uint32_t)a.s_tok_b);
                    L.nreal = uniform(min(max(t1 - tw, 0), kTokPerWave));
                }
                return L;
            };
            // row of token tt of the wave's 8 relative to its first (two groups of 4)
            auto tok_row = [](int tt) { return (tt >> 2) * kHalfGroupBytes + (tt & 3) * kRowStep; };
            auto dma_token = [&](const TileLoads &L, int tt) {
                if (SPARSE) {
                    const bool ok = (L.nreal >> tt) & 1;
                    if (lane < kChunks) lds_dma_buf16(a.k_pool + L.toff[tt], ok ? kTokBytes : 0, 16 * lane, L.lds0 + tok_row(tt));
                } else {
                    // (a buffer per token: the range check of a buffer load leaves out the
                    // scalar offset, so a token past the real ones needs a buffer of its own)
                    if (lane < kChunks)
                        lds_dma_buf16(L.tok + tt * (uint32_t)a.s_tok_b, tt < L.nreal ? kTokBytes : 0, 16 * lane,
                                      L.lds0 + tok_row(tt));
                }
            };
            auto end_tile = [&](int t) {
                if (!SPARSE) dn_issue_page(t + kAhead);
            };
            auto issue_tile = [&](int t, int page) {
                const TileLoads L = prep_tile(t, page);
#pragma unroll
                for (int tt = 0; tt < kTokPerWave; tt++) dma_token(L, tt);
                end_tile(t);
            };

            // ---- top of tile i (all waves, same barriers): each value wave waits for its
            //      loads of tile i+1 (tiles up to i+kAhead-1 are in flight, the younger one may
            //      stay), all waves are past tile i-1 (slot of tile i-2 free, the B operands and
            //      half maxima of tile i-1's iteration stored); returns where the loads of tile
            //      i+kAhead go (each value wave issues exactly one tile's loads per iteration,
            //      which the wait counts rely on)
            auto tile_top = [&](int i) {
                wait_vmcnt<(kAhead - 2) * kLoadsPerTile>();
                if (SPARSE) {
                    lds_barrier();
                    return prep_tile(i + kAhead, 0);
                } else {
                    return prep_tile(i + kAhead, page_barrier(i + kAhead));
                }
            };

            if (ntiles > 0) {
                // ---- prologue: lookups (sparse), the loads of tiles 0..kAhead-1; tile 0 in
                {
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
                    wait_vmcnt<(kAhead - 1) * kLoadsPerTile>();
                }
                lds_barrier();
            }

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
                // V^T of the tile: blocks 0 and 1 read before the barrier, block d + 2 while the
                // MFMAs of block d run; A = V^T converted one block ahead
                i32x2 vw[3];
                for (int i = 0; ntiles > 0 && i <= ntiles; i++) {
                    const TileLoads ld = tile_top(i);
                    if (i == 0) {
#pragma unroll
                        for (int tt = 0; tt < kTokPerWave; tt++) dma_token(ld, tt);
                    }
                    if (i > 0) {
                        const int j = i - 1;
                        PA_LDS uint8_t *vb = vbase(j);
                        // the tile's factors for O^T and the B operands (P^T of head block hb
                        // times value tile vt's token scales, from the score waves of hb)
                        bf16x8 pbt[4];
#pragma unroll
                        for (int hb = 0; hb < 4; hb++) {
                            const bf16x4 lo = s_p[j & 1][hb][vt][0][lane], hi = s_p[j & 1][hb][vt][1][lane];
#pragma unroll
                            for (int k = 0; k < 4; k++) {
                                pbt[hb][k] = lo[k];
                                pbt[hb][4 + k] = hi[k];
                            }
                        }
                        {
                            float alpha[4];
#pragma unroll
                            for (int hb = 0; hb < 4; hb++) alpha[hb] = s_alpha[j & 1][hb][col];
                            if (__any(alpha[0] != 1.f || alpha[1] != 1.f || alpha[2] != 1.f || alpha[3] != 1.f)) {
                                mfma_acc_drain(acc);             // rare: a reference moved
#pragma unroll
                                for (int d = 0; d < kDvBlocks; d++) acc[d] = acc[d] * alpha[d & 3];
                                mfma_acc_drain(acc);             // (wait states before the MFMAs)
                            }
                        }
                        vw[2] = rd(vb, 2);
                        bf16x8 va[2];
                        va[0] = fp8x8_to_bf16((uint32_t)vw[0][0], (uint32_t)vw[0][1]);
                        asm volatile("s_nop 1" : "+v"(va[0]));
#pragma unroll
                        for (int d = 0; d < kVBlocks; d++) {
#pragma unroll
                            for (int hb = 0; hb < 4; hb++) mfma_acc(acc[4 * d + hb], va[d & 1], pbt[hb]);
                            dma_token(ld, d);              // token d of tile i + kAhead
                            if (d + 3 < kVBlocks) vw[d % 3] = rd(vb, d + 3);
                            if (d + 1 < kVBlocks) {
                                va[(d + 1) & 1] = fp8x8_to_bf16((uint32_t)vw[(d + 1) % 3][0], (uint32_t)vw[(d + 1) % 3][1]);
                                // wait states between this VALU write and the next block's MFMAs,
                                // which the compiler does not see (asm)
                                asm volatile("s_nop 1" : "+v"(va[(d + 1) & 1]));
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    end_tile(i + kAhead);
                    if (i < ntiles) {
                        PA_LDS uint8_t *vbn = vbase(i);
                        vw[0] = rd(vbn, 0);
                        vw[1] = rd(vbn, 1);
                    }
                }
                mfma_acc_drain(acc);
                lds_barrier();                                   // both halves' sums
                lds_barrier();                                   // s_inv in
                // ---- epilogue: rows of head block hb: draft token and heads as in the score wave
                // (the lane's column is made opaque here, so that the row addresses are worked
                // out per item instead of being kept, and spilled, across the whole loop)
                int ecol = col;
                asm volatile("" : "+v"(ecol));
#pragma unroll
                for (int hb = 0; hb < 4; hb++) {
                    const int r0 = group * kHeadsPerWG + hb * kHeadsPerWave;
                    if (r0 >= G * nq) continue;                  // no query rows
                    const int q_i = r0 / G;
                    const int64_t row = (int64_t)q_i * Hq + (r0 - q_i * G) + ecol;
                    const float inv = s_inv[hb][ecol];
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
                            // (a buffer over the item's partial rows; `it` is uniform)
                            const __amdgpu_buffer_rsrc_t rows =
                                shared_rows(a.ws_o + (int64_t)it * nq * Hq * kDv, (int64_t)nq * Hq * kDv * 4);
                            const uint32_t off = (uint32_t)((row * kDv + 128 * vt + 4 * g4) * 4);
#pragma unroll
                            for (int d = 0; d < kVBlocks; d++) store_shared4(rows, off + 64 * d, acc[4 * d + hb] * inv);
                        } else {
#pragma unroll
                            for (int d = 0; d < kVBlocks; d++) *(f32x4 *)(orow + 16 * d) = acc[4 * d + hb] * inv;
                        }
                    }
                }
            lds_barrier();                                   // the item's LDS is free
        }
    }
    // fused combine (dense, one query token: the head group is heads [64 group, 64 group +
    // 64)): the last workgroup to finish a request's chunks merges them, two units per
    // thread and pass (768 threads; four spill registers in the main loops)
    if (!SPARSE && a.counters)
        fused_combine_tail<2>(a, plan, part, ib, ie, group, ngroups, group * kHeadsPerWG,
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
