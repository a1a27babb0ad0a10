// Split-KV paged decode kernel for bf16 and fp8-e4m3 (per page and KV head scale) KV,
// head dims 64 and 128, up to 16 query heads per KV head, gfx950.
//
// One workgroup = one (part, KV head); it walks the part's items (request, token
// range).  Its 4 waves take the item's token blocks round robin and work
// independently - every wave keeps its own online-softmax state - then merge
// through LDS at the end of the item (the split-KV merge of the XQA article,
// section "归约怎么记", applied across waves).
//
// Per token block (BT = 16 or 32 tokens, 8 KiB of K+V at D = 128) and wave, in the
// S^T orientation (SWAP_AB in the XQA article's terms, section "SWAP_AB: 把 K 放在
// A 位"):
//   S^T[16 tok x 16 heads] = K[16 tok x D] . Q^T[D x 16 heads]: bf16 MFMA 16x16x32
//       chains; K goes from HBM straight into the MFMA A operand (16 B per lane,
//       the token row of lane%16), Q^T stays in registers (query rows padded from
//       G to 16 with zeros; XQA article, section "GQA 的组内复用").
//   online softmax per head column in the log2 domain (exp(x) = 2^(x log2 e),
//       pipelining page, section 一); block max across the 4 lane groups with
//       shuffles.  The C layout of S^T is the B operand layout P^T needs.
//   O^T[D x 16 heads] += V^T[D x BT tok] . P^T[BT tok x 16 heads]: V goes through a
//       wave-private LDS tile and comes back transposed with ds_read_b64_tr_b16
//       (bf16) or ds_read_b64_tr_b8 + e4m3->bf16 conversion (fp8).
// Loads run NB-1 blocks ahead of the compute through a ring of register buffers
// (the load/compute overlap of the pipelining page, section "除了计算，还有搬运").
// FP8 K/V are converted to bf16 exactly in registers; the K scale of a page
// multiplies that page's logits, the V scale multiplies P before the PV product
// (XQA article, section "FP8 / INT8 的 KV: 转换到底放在哪儿", scale folding).
//
// Several query tokens per request (a linear speculative draft; XQA article, section
// "投机解码: XQA 的第二个工作负载", which folds draft tokens x GQA heads into the MMA
// row dimension): the G * q_len query rows of a KV head fill the 16 MFMA columns, more
// than 16 rows take several column tiles (grid z).  Column (qi, g) masks the keys past
// its causal limit L - q_len + qi + 1.
#include "pa_merge.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// Cache policy bits of the KV buffer loads.  2 = non-temporal: every KV byte is read
// exactly once, so streaming it past the caches keeps them for the tables and partials
// (the analogue of the evict-first hint in the FlashMLA walk-through, section 数据加载);
// measured +11% bandwidth over the default policy on the Llama-70B-like workload.
#ifndef PA_KV_LOAD_AUX
#define PA_KV_LOAD_AUX 2
#endif
// Register ring depth (blocks) and the token-row byte threshold at or above which a
// wave iteration covers 16 tokens instead of 32.  Depth 2 (one block in flight while one
// is computed) measured fastest on MI355X: 191 registers instead of 254 at depth 4, and
// -4 % time on the ragged FP8 workload, -1.5 % on the bf16 one.
#ifndef PA_RING_DEPTH
#define PA_RING_DEPTH 2
#endif
#ifndef PA_BT16_MIN_ROW_BYTES
#define PA_BT16_MIN_ROW_BYTES 256
#endif

template <int D, bool FP8>
struct Cfg {
    static constexpr int EB = FP8 ? 1 : 2;            // stored bytes per element
    static constexpr int ROWB = D * EB;               // bytes of one token row
    static constexpr int BT = ROWB >= PA_BT16_MIN_ROW_BYTES ? 16 : 32;  // tokens per wave iteration
    static constexpr int NSB = BT / 16;               // 16-token MFMA row blocks per iteration
    static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
    static constexpr int NLD = CPR / 4;               // K (and V) loads per lane per sub-block
    static constexpr int NS = D / 32;                 // k-steps of the QK^T MFMA chain
    static constexpr int NDB = D / 16;                // 16-dim blocks of the PV MFMA
    static constexpr int RS = ROWB + 16;              // LDS row stride of the V tile (padded)
    static constexpr int VTILE = BT * RS;             // bytes of one wave's V tile
    static constexpr int NB = PA_RING_DEPTH;          // register ring depth (blocks)
    static_assert(CPR % 4 == 0, "row must split over 4 lane groups");
    static_assert(!FP8 || BT == 32, "fp8 PV uses the k = 32 MFMA");
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// e4m3 x4 (one dword) -> bf16 x4, exact (gfx950 OCP fp8 conversion, scale 1).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1)
{
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

template <typename T>
__device__ __forceinline__ T lds_tr(const uint8_t *p);

template <>
__device__ __forceinline__ bf16x4 lds_tr<bf16x4>(const uint8_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4 *)((__attribute__((address_space(3))) uint8_t *)p));
}

template <>
__device__ __forceinline__ i32x2 lds_tr<i32x2>(const uint8_t *p)
{
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2 *)((__attribute__((address_space(3))) uint8_t *)p));
}

template <int D, bool FP8>
struct BlockRegs {
    u32x4 k[Cfg<D, FP8>::NSB][Cfg<D, FP8>::NLD];   // K rows, per 16-token sub-block
    u32x4 v[Cfg<D, FP8>::NSB * Cfg<D, FP8>::NLD];  // V chunks (row-major chunk order)
    float ks[Cfg<D, FP8>::NSB], vs[Cfg<D, FP8>::NSB];  // fp8 page scales
};

// Raw buffer resource over `nbytes` bytes at a wave-uniform base: loads through it take
// a 32-bit per-lane offset (one VGPR instead of a 64-bit address) and read 0 past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t *base, int nbytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, nbytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, PA_KV_LOAD_AUX);
}

// Issue the loads of the block starting at token tb (tb < t1).  A sub-block that
// starts at or beyond t1 reloads the first sub-block's rows (an L2 hit) so that every
// block issues the same number of loads; its tokens are masked when processed.
// koff / voff are the lane's byte offsets inside a 16-token sub-block (see the kernel).
template <int D, bool FP8>
__device__ __forceinline__ void load_block(const DecodeArgs &a, const int32_t *__restrict__ bt,
                                           const float *__restrict__ ksc,
                                           const float *__restrict__ vsc, int b, int h, int tb,
                                           int t1, int koff, int voff, BlockRegs<D, FP8> &r)
{
    using C = Cfg<D, FP8>;
    const int span = 16 * (int)a.s_tok_b;            // bytes covering 16 token rows
#pragma unroll
    for (int sb = 0; sb < C::NSB; sb++) {
        const int ts = tb + 16 * sb < t1 ? tb + 16 * sb : tb;
        const int page = bt[(int64_t)b * a.max_pages + (ts >> a.page_shift)];
        const int slot = ts & ((1 << a.page_shift) - 1);
        const int64_t base = (int64_t)page * a.s_page_b + (int64_t)h * a.s_head_b +
                             (int64_t)slot * a.s_tok_b;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.k_pool + base, span);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(a.v_pool + base, span);
#pragma unroll
        for (int u = 0; u < C::NLD; u++) r.k[sb][u] = bload(kr, koff + 64 * u, 0);
#pragma unroll
        for (int u = 0; u < C::NLD; u++)
            r.v[sb * C::NLD + u] = bload(vr, voff, u * (64 / C::CPR) * (int)a.s_tok_b);
        if (FP8) {
            r.ks[sb] = ksc[(int64_t)page * a.Hkv + h];
            r.vs[sb] = vsc[(int64_t)page * a.Hkv + h];
        } else {
            r.ks[sb] = 1.0f;
            r.vs[sb] = 1.0f;
        }
    }
}

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void pa_decode_kernel(
    DecodeArgs a, const int32_t *__restrict__ plan, const int32_t *__restrict__ bt,
    const float *__restrict__ ksc, const float *__restrict__ vsc,
    const int32_t *__restrict__ seq_lens)
{
    // read-only tables come in as separate restrict arguments so that their wave-uniform
    // reads compile to scalar loads (a vector load would join the in-order vmcnt queue)
    using C = Cfg<D, FP8>;
    constexpr int BT = C::BT, NB = C::NB;
    constexpr int kLdsV = kWaves * C::VTILE;
    constexpr int kLdsO = kWaves * D * 17 * 4;        // epilogue: per-wave O^T, padded
    constexpr int kLds = kLdsV > kLdsO ? kLdsV : kLdsO;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];
    __shared__ float s_M[16], s_L[16];
    __shared__ int s_flag;

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int col = lane & 15, g4 = lane >> 4;
    const int part = blockIdx.x, h = blockIdx.y;
    const int G = a.G, Hq = a.Hkv * a.G, nq = a.q_len, rows = G * nq;
    // this lane's MFMA column: query row c = 16 * blockIdx.z + col = qi * G + g
    const int c = 16 * blockIdx.z + col;
    const int cqi = c / G, cg = c - (c / G) * G;
    uint8_t *vt = lds + wave * C::VTILE;
    // lane byte offsets inside a 16-token sub-block: K row `col`, 16-byte chunk g4 (+4u);
    // V chunk `lane` of the row-major chunk order (row lane / CPR, chunk lane % CPR)
    const int koff = col * (int)a.s_tok_b + g4 * 16;
    const int voff = (lane / C::CPR) * (int)a.s_tok_b + (lane % C::CPR) * 16;

    // a fixed-split plan has exactly one item per part (no plan read on the critical path)
    const int ib = a.fixed_splits > 0 ? part : plan[a.part_begin_off + part];
    const int ie = a.fixed_splits > 0 ? part + 1 : plan[a.part_begin_off + part + 1];

    for (int it = ib; it < ie; it++) {
        const int b = plan[a.items_off + 4 * it + 0];
        const int t0 = plan[a.items_off + 4 * it + 1];
        const int t1 = plan[a.items_off + 4 * it + 2];
        const int flags = plan[a.items_off + 4 * it + 3];

        // ---- Q^T operand (B of the QK MFMA): lane holds query row c, 8 dims per k-step
        bf16x8 qop[C::NS];
        {
            const uint16_t *qrow = a.q + (((int64_t)b * nq + cqi) * Hq + (int64_t)h * G + cg) * D;
#pragma unroll
            for (int s = 0; s < C::NS; s++) {
                const int d0 = FP8 ? 16 * (4 * (s >> 1) + g4) + 8 * (s & 1) : 8 * (4 * s + g4);
                if (c < rows)
                    qop[s] = *(const bf16x8 *)(qrow + d0);
                else
                    qop[s] = bf16x8{};
            }
        }
        // keys this column may see in the item: [max(t0, tlo), tlim): the causal limit of
        // its query token (every key of the item when q_len = 1) and the sliding window
        int tlim = t1, tlo = 0;
        if (nq > 1 || a.window > 0) {
            const int L = seq_lens[b];
            if (nq > 1) tlim = min(t1, L - (nq - 1 - cqi));
            if (a.window > 0) tlo = max(0, L - nq + cqi - a.window + 1);
        }

        float m = -INFINITY;      // running max (log2 domain) of head `col`
        float l = 0.f;            // this lane's share of the denominator
        f32x4 acc[C::NDB];
#pragma unroll
        for (int i = 0; i < C::NDB; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

        // this wave's blocks: wave, wave + 4, ...; block i starts at token t0 + BT*(wave + 4i)
        const int nblk = (t1 - t0 + BT - 1) / BT;
        const int nmine = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
        auto block_tb = [&](int i) {
            const int ic = i < nmine ? i : nmine - 1;     // past the end: reload the last block
            return t0 + BT * (wave + kWaves * ic);
        };

        if (nmine > 0) {
            BlockRegs<D, FP8> ring[NB];
#pragma unroll
            for (int p = 0; p < NB - 1; p++) load_block<D, FP8>(a, bt, ksc, vsc, b, h, block_tb(p), t1, koff, voff, ring[p]);

            // The wave's block count is rounded up to a multiple of NB: the ring loop then
            // has no early exit, which keeps the compiler's vmcnt waits exact (only the
            // current block's loads are waited for).  Blocks past the wave's last one
            // (i >= nmine) reload that last block and are processed fully masked.
            for (int i0 = 0; i0 < nmine; i0 += NB) {
#pragma unroll
                for (int u = 0; u < NB; u++) {
                    const int i = i0 + u;
                    load_block<D, FP8>(a, bt, ksc, vsc, b, h, block_tb(i + NB - 1), t1, koff, voff,
                                      ring[(u + NB - 1) % NB]);
                    const BlockRegs<D, FP8> &cur = ring[u];
                    const int tb = t0 + BT * (wave + kWaves * i);

                    // ---- V rows into the wave's LDS tile; rows of tokens >= t1 become 0 so
                    //      that masked probabilities (0) never meet non-finite padding data
#pragma unroll
                    for (int sb = 0; sb < C::NSB; sb++) {
#pragma unroll
                        for (int uu = 0; uu < C::NLD; uu++) {
                            const int x = uu * 64 + lane;
                            const int tt = x / C::CPR, c = x % C::CPR;
                            const int row = 16 * sb + tt;
                            u32x4 v = cur.v[sb * C::NLD + uu];
                            if (tb + row >= t1) v = u32x4{0, 0, 0, 0};
                            *(u32x4 *)(vt + row * C::RS + c * 16) = v;
                        }
                    }

                    // ---- S^T = K . Q^T per 16-token sub-block
                    f32x4 st[C::NSB];
#pragma unroll
                    for (int sb = 0; sb < C::NSB; sb++) {
                        f32x4 c4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int uu = 0; uu < C::NLD; uu++) {
                            const u32x4 w = cur.k[sb][uu];
                            if (FP8) {
                                c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    e4m3x8_to_bf16(w[0], w[1]), qop[2 * uu], c4, 0, 0, 0);
                                c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    e4m3x8_to_bf16(w[2], w[3]), qop[2 * uu + 1], c4, 0, 0, 0);
                            } else {
                                c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, w), qop[uu], c4, 0, 0, 0);
                            }
                        }
                        st[sb] = c4;
                    }

                    // ---- online softmax (per head column; tokens 16*sb + 4*g4 + r)
                    float sv[C::NSB][4];
                    float bm = -INFINITY;
#pragma unroll
                    for (int sb = 0; sb < C::NSB; sb++) {
                        const float f = a.scale_log2 * cur.ks[sb];
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const int tok = tb + 16 * sb + 4 * g4 + r;
                            const float x = st[sb][r] * f;
                            sv[sb][r] = (tok < tlim && tok >= tlo) ? x : -INFINITY;
                            bm = fmaxf(bm, sv[sb][r]);
                        }
                    }
                    bm = fmaxf(bm, __shfl_xor(bm, 16));
                    bm = fmaxf(bm, __shfl_xor(bm, 32));
                    const float mn = fmaxf(m, bm);
                    const float mref = mn == -INFINITY ? 0.f : mn;
                    // a column with no visible key yet (its query token's causal limit) keeps
                    // alpha = 1: its state is still zero
                    const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mref);
                    m = mn;
                    __bf16 pbv[4 * C::NSB];
                    float ps = 0.f;
#pragma unroll
                    for (int sb = 0; sb < C::NSB; sb++) {
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            // the denominator takes the fp32 weight: summing the bf16-rounded
                            // weights moves lse by up to ~2^-9 when a few keys dominate
                            const float p = fast_exp2(sv[sb][r] - mref);
                            ps += p;
                            pbv[4 * sb + r] = (__bf16)(FP8 ? p * cur.vs[sb] : p);
                        }
                    }
                    l = l * alpha + ps;
                    if (__any(alpha != 1.f)) {
#pragma unroll
                        for (int db = 0; db < C::NDB; db++) acc[db] *= alpha;
                    }

                    // ---- O^T += V^T . P^T (V^T operand read back transposed from LDS)
                    const int jj = lane & 15;
#pragma unroll
                    for (int db = 0; db < C::NDB; db++) {
                        if (FP8) {
                            // 8 tokens per lane: k = 8*g4 + r <-> token (r < 4 ? 4g4+r : 16+4g4+r-4)
                            const int rr = jj >> 1;
                            const int tok = rr < 4 ? 4 * g4 + rr : 16 + 4 * g4 + (rr - 4);
                            const i32x2 w = lds_tr<i32x2>(vt + tok * C::RS + 16 * db + 8 * (jj & 1));
                            bf16x8 pb;
#pragma unroll
                            for (int k = 0; k < 8; k++) pb[k] = pbv[k];
                            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                e4m3x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]), pb, acc[db], 0, 0, 0);
                        } else if (BT == 32) {
                            const int rr = jj >> 2;
                            const bf16x4 lo =
                                lds_tr<bf16x4>(vt + (4 * g4 + rr) * C::RS + (16 * db + 4 * (jj & 3)) * 2);
                            const bf16x4 hi =
                                lds_tr<bf16x4>(vt + (16 + 4 * g4 + rr) * C::RS + (16 * db + 4 * (jj & 3)) * 2);
                            bf16x8 va, pb;
#pragma unroll
                            for (int k = 0; k < 4; k++) {
                                va[k] = lo[k];
                                va[4 + k] = hi[k];
                            }
#pragma unroll
                            for (int k = 0; k < 8; k++) pb[k] = pbv[k];
                            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[db], 0, 0, 0);
                        } else {
                            // 16-token block: k = 4*g4 + r <-> token 4*g4 + r
                            const int rr = jj >> 2;
                            const bf16x4 va =
                                lds_tr<bf16x4>(vt + (4 * g4 + rr) * C::RS + (16 * db + 4 * (jj & 3)) * 2);
                            bf16x4 pb;
#pragma unroll
                            for (int k = 0; k < 4; k++) pb[k] = pbv[k];
                            acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                                __builtin_bit_cast(s16x4, va), __builtin_bit_cast(s16x4, pb), acc[db], 0, 0, 0);
                        }
                    }
                }
            }
        }

        // ---- merge the 4 waves' states through LDS
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (lane < 16) {
            s_m[wave][lane] = m;
            s_l[wave][lane] = l;
        }
        __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmaxf(M, s_m[w][col]);
        float Lt = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float mw = s_m[w][col];
            if (mw != -INFINITY) Lt += s_l[w][col] * fast_exp2(mw - M);
        }
        if (a.sinks && (flags & 1) && c < rows) {
            // the item is the whole request: its sink joins the denominator here (split
            // requests get it in the merge)
            const float sk = a.sinks[h * G + cg] * 1.4426950408889634f;
            const float M2 = fmaxf(M, sk);
            if (M2 != -INFINITY) {
                Lt = (M == -INFINITY ? 0.f : Lt * fast_exp2(M - M2)) + fast_exp2(sk - M2);
                M = M2;
            }
        }
        const float f = (m == -INFINITY || Lt == 0.f) ? 0.f : fast_exp2(m - M) / Lt;
        if (wave == 0 && lane < 16) {
            s_M[lane] = M;
            s_L[lane] = Lt;
        }
        float *so = (float *)lds;                       // [wave][dim][17] (padded head axis)
#pragma unroll
        for (int db = 0; db < C::NDB; db++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                so[(wave * D + 16 * db + 4 * g4 + r) * 17 + col] = acc[db][r] * f;
        __syncthreads();

        // ---- write: 8 consecutive dims of one query row (column `head`) per thread
        {
            const int t = threadIdx.x;
            const int head = t / (D / 8), d0 = (t % (D / 8)) * 8;
            const int cr = 16 * blockIdx.z + head;
            if (cr < rows && t < 16 * (D / 8)) {
                float o[8];
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    float s = 0.f;
#pragma unroll
                    for (int w = 0; w < kWaves; w++) s += so[(w * D + d0 + k) * 17 + head];
                    o[k] = s;
                }
                const float Mh = s_M[head], Lh = s_L[head];
                const float lse_v = (Mh == -INFINITY || Lh == 0.f)
                                        ? -INFINITY
                                        : (Mh + log2f(Lh)) * 0.69314718055994530942f;
                const int qi = cr / G;
                const int64_t qr = (int64_t)qi * Hq + (int64_t)h * G + (cr - qi * G);
                const int64_t row = (int64_t)b * nq * Hq + qr;
                if (flags & 1) {
                    bf16x8 ob;
#pragma unroll
                    for (int k = 0; k < 8; k++) ob[k] = (__bf16)o[k];
                    *(bf16x8 *)(a.out + row * a.Dv + d0) = ob;
                    if (d0 == 0) a.lse[row] = lse_v;
                } else {
                    const int64_t prow = (int64_t)it * nq * Hq + qr;
                    float *dst = a.ws_o + prow * a.Dv + d0;
                    if (a.counters) {                 // merged inside this launch
                        // (a buffer over the item's partial rows; `it` is uniform)
                        const int64_t prow0 = (int64_t)it * nq * Hq;
                        const __amdgpu_buffer_rsrc_t rows = shared_rows(a.ws_o + prow0 * a.Dv, (int64_t)nq * Hq * a.Dv * 4);
                        const uint32_t off = (uint32_t)(((prow - prow0) * a.Dv + d0) * 4);
                        store_shared4(rows, off, merge_f32x4{o[0], o[1], o[2], o[3]});
                        store_shared4(rows, off + 16, merge_f32x4{o[4], o[5], o[6], o[7]});
                        if (d0 == 0) store_shared(a.ws_lse + prow, lse_v);
                    } else {
                        *(f32x4 *)dst = f32x4{o[0], o[1], o[2], o[3]};
                        *(f32x4 *)(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
                        if (d0 == 0) a.ws_lse[prow] = lse_v;
                    }
                }
            }
        }
        __syncthreads();
    }
    // fused combine: the last workgroup to finish a request's chunks merges them
    if (a.counters)
        fused_combine_tail<2>(a, plan, part, ib, ie, h, a.Hkv, h * G, G, gridDim.z, &s_flag);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    const dim3 grid(a.num_parts, a.Hkv, (a.G * a.q_len + 15) / 16), block(kThreads);
    const bool fp8 = a.kv_format == PA_KV_FP8_E4M3_PAGE_HEAD;
    if (a.D == 128 && !fp8)
        hipLaunchKernelGGL((pa_decode_kernel<128, false>), grid, block, 0, stream, a, a.plan,
                           a.block_table, a.k_scale, a.v_scale, a.seq_lens);
    else if (a.D == 64 && !fp8)
        hipLaunchKernelGGL((pa_decode_kernel<64, false>), grid, block, 0, stream, a, a.plan,
                           a.block_table, a.k_scale, a.v_scale, a.seq_lens);
    else if (a.D == 128 && fp8)
        hipLaunchKernelGGL((pa_decode_kernel<128, true>), grid, block, 0, stream, a, a.plan,
                           a.block_table, a.k_scale, a.v_scale, a.seq_lens);
    else if (a.D == 64 && fp8)
        hipLaunchKernelGGL((pa_decode_kernel<64, true>), grid, block, 0, stream, a, a.plan,
                           a.block_table, a.k_scale, a.v_scale, a.seq_lens);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
