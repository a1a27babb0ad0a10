// Split-KV paged decode kernel for bf16 and fp8-e4m3 (per page and KV head scale) KV,
// head dims 64 and 128, up to 16 query heads per KV head, gfx950.
//
// One workgroup = one (part, KV head); it walks the part's items (request, token
// range).  Its 4 waves split each item's 32-token blocks round robin and work
// independently - every wave keeps its own online-softmax state - then merge
// through LDS at the end of the item (the split-KV merge of the XQA article,
// section "归约怎么记", applied across waves).
//
// Per 32-token block and wave (S^T orientation, SWAP_AB in the XQA article's terms,
// section "SWAP_AB: 把 K 放在 A 位"):
//   S^T[16 tok x 16 heads] = K[16 tok x D] . Q^T[D x 16 heads]  two bf16 MFMA
//       16x16x32 chains; K is loaded from HBM straight into the MFMA A operand
//       (16 B per lane, the token row of lane%16), Q^T is resident in registers
//       (query rows padded from G to 16 with zeros, XQA section "GQA 的组内复用").
//   online softmax per head column in the log2 domain (exp(x) = 2^(x log2 e),
//       pipelining page, section 一), block max across the 4 lane groups with
//       shuffles.  The C layout of S^T is exactly the B operand layout P^T needs.
//   O^T[D x 16 heads] += V^T[D x 32 tok] . P^T[32 tok x 16 heads]: V goes through a
//       wave-private LDS tile and comes back transposed with ds_read_b64_tr_b16
//       (bf16) or ds_read_b64_tr_b8 + e4m3->bf16 conversion (fp8).
// FP8 K/V are converted to bf16 exactly in registers; the K scale of a page
// multiplies that page's logits, the V scale multiplies P before the PV product
// (XQA article, section "FP8 / INT8 的 KV: 转换到底放在哪儿", scale folding).
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockTok = 32;     // tokens per wave iteration (two 16-token MFMA row blocks)

template <int D, bool FP8>
struct Cfg {
    static constexpr int EB = FP8 ? 1 : 2;            // stored bytes per element
    static constexpr int ROWB = D * EB;               // bytes of one token row
    static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
    static constexpr int NLD = CPR / 4;               // K loads per lane per 16-token sub-block
    static constexpr int NS = D / 32;                 // k-steps of the QK^T MFMA chain
    static constexpr int NDB = D / 16;                // 16-dim blocks of the PV MFMA
    static constexpr int RS = ROWB + 16;              // LDS row stride of the V tile (padded)
    static constexpr int VTILE = kBlockTok * RS;      // bytes of one wave's V tile
    static constexpr int NVLD = 2 * NLD;              // V loads per lane per block
    static_assert(CPR % 4 == 0, "row must split over 4 lane groups");
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// e4m3 x4 (one dword) -> bf16 x4, exact (gfx950 OCP fp8 conversion, scale 1).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, bf16x2 &lo, bf16x2 &hi)
{
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1)
{
    bf16x2 a, b, c, d;
    e4m3x4_to_bf16(w0, a, b);
    e4m3x4_to_bf16(w1, c, d);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

template <int D, bool FP8>
struct BlockRegs {
    u32x4 k[2][Cfg<D, FP8>::NLD];     // K rows, per 16-token sub-block
    u32x4 v[Cfg<D, FP8>::NVLD];       // V chunks (row-major chunk order of the block)
    float ks[2], vs[2];               // fp8 page scales of the two sub-blocks
    int valid[2];                     // sub-block has at least one token < t1
};

template <int D, bool FP8>
__device__ __forceinline__ void load_block(const DecodeArgs &a, int b, int h, int tb, int t1,
                                           int lane, BlockRegs<D, FP8> &r)
{
    using C = Cfg<D, FP8>;
    const int col = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int sb = 0; sb < 2; sb++) {
        const int ts = tb + 16 * sb;
        r.valid[sb] = ts < t1;
        r.ks[sb] = 1.0f;
        r.vs[sb] = 1.0f;
        if (ts < t1) {
            const int page = a.block_table[(int64_t)b * a.max_pages + (ts >> a.page_shift)];
            const int slot = ts & ((1 << a.page_shift) - 1);
            const int64_t base = (int64_t)page * a.s_page_b + (int64_t)h * a.s_head_b +
                                 (int64_t)slot * a.s_tok_b;
            const uint8_t *kp = a.k_pool + base + (int64_t)col * a.s_tok_b;
#pragma unroll
            for (int u = 0; u < C::NLD; u++)
                r.k[sb][u] = *(const u32x4 *)(kp + (4 * u + g4) * 16);
            const uint8_t *vp = a.v_pool + base;
#pragma unroll
            for (int u = 0; u < C::NLD; u++) {
                const int x = u * 64 + lane;
                const int tt = x / C::CPR, c = x % C::CPR;
                r.v[sb * C::NLD + u] = *(const u32x4 *)(vp + (int64_t)tt * a.s_tok_b + c * 16);
            }
            if (FP8) {
                r.ks[sb] = a.k_scale[(int64_t)page * a.Hkv + h];
                r.vs[sb] = a.v_scale[(int64_t)page * a.Hkv + h];
            }
        } else {
#pragma unroll
            for (int u = 0; u < C::NLD; u++) {
                r.k[sb][u] = u32x4{0, 0, 0, 0};
                r.v[sb * C::NLD + u] = u32x4{0, 0, 0, 0};
            }
        }
    }
}

// Write the block's V rows into the wave's LDS tile; rows of tokens >= t1 become 0 so
// that masked probabilities (0) never meet non-finite padding data.
template <int D, bool FP8>
__device__ __forceinline__ void store_v(uint8_t *vt, const BlockRegs<D, FP8> &r, int tb, int t1,
                                        int lane)
{
    using C = Cfg<D, FP8>;
#pragma unroll
    for (int sb = 0; sb < 2; sb++) {
#pragma unroll
        for (int u = 0; u < C::NLD; u++) {
            const int x = u * 64 + lane;
            const int tt = x / C::CPR, c = x % C::CPR;
            const int row = 16 * sb + tt;
            u32x4 v = r.v[sb * C::NLD + u];
            if (tb + row >= t1) v = u32x4{0, 0, 0, 0};
            *(u32x4 *)(vt + row * C::RS + c * 16) = v;
        }
    }
}

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) void pa_decode_kernel(DecodeArgs a)
{
    using C = Cfg<D, FP8>;
    constexpr int kLdsV = kWaves * C::VTILE;
    constexpr int kLdsO = kWaves * D * 17 * 4;        // epilogue: per-wave O^T, padded
    constexpr int kLds = kLdsV > kLdsO ? kLdsV : kLdsO;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];
    __shared__ float s_M[16], s_L[16];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int col = lane & 15, g4 = lane >> 4;
    const int part = blockIdx.x, h = blockIdx.y;
    const int G = a.G, Hq = a.Hkv * a.G;
    uint8_t *vt = lds + wave * C::VTILE;

    const int ib = a.plan[a.part_begin_off + part];
    const int ie = a.plan[a.part_begin_off + part + 1];

    for (int it = ib; it < ie; it++) {
        const int b = a.plan[a.items_off + 4 * it + 0];
        const int t0 = a.plan[a.items_off + 4 * it + 1];
        const int t1 = a.plan[a.items_off + 4 * it + 2];
        const int flags = a.plan[a.items_off + 4 * it + 3];

        // ---- Q^T operand (B of the QK MFMA): lane holds head `col`, 8 dims per k-step
        bf16x8 qop[C::NS];
        {
            const uint16_t *qrow = a.q + ((int64_t)b * Hq + (int64_t)h * G + col) * D;
#pragma unroll
            for (int s = 0; s < C::NS; s++) {
                const int d0 = FP8 ? 16 * (4 * (s >> 1) + g4) + 8 * (s & 1) : 8 * (4 * s + g4);
                if (col < G)
                    qop[s] = *(const bf16x8 *)(qrow + d0);
                else
                    qop[s] = bf16x8{};
            }
        }

        float m = -INFINITY;      // running max (log2 domain) of head `col`
        float l = 0.f;            // this lane's share of the denominator
        f32x4 acc[C::NDB];
#pragma unroll
        for (int i = 0; i < C::NDB; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

        const int nblk = (t1 - t0 + kBlockTok - 1) / kBlockTok;
        BlockRegs<D, FP8> cur, nxt;
        int j = wave;
        if (j < nblk) load_block<D, FP8>(a, b, h, t0 + kBlockTok * j, t1, lane, cur);

        for (; j < nblk; j += kWaves) {
            const int tb = t0 + kBlockTok * j;
            store_v<D, FP8>(vt, cur, tb, t1, lane);
            if (j + kWaves < nblk)
                load_block<D, FP8>(a, b, h, tb + kBlockTok * kWaves, t1, lane, nxt);

            // ---- S^T = K . Q^T for the two 16-token sub-blocks
            f32x4 st[2];
#pragma unroll
            for (int sb = 0; sb < 2; sb++) {
                f32x4 c4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < C::NLD; u++) {
                    const u32x4 w = cur.k[sb][u];
                    if (FP8) {
                        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(w[0], w[1]),
                                                                     qop[2 * u], c4, 0, 0, 0);
                        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(w[2], w[3]),
                                                                     qop[2 * u + 1], c4, 0, 0, 0);
                    } else {
                        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, w), qop[u], c4, 0, 0, 0);
                    }
                }
                st[sb] = c4;
            }

            // ---- online softmax (per head column; tokens 16*sb + 4*g4 + r)
            float sv[2][4];
            float bm = -INFINITY;
#pragma unroll
            for (int sb = 0; sb < 2; sb++) {
                const float f = a.scale_log2 * cur.ks[sb];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int tok = tb + 16 * sb + 4 * g4 + r;
                    const float x = st[sb][r] * f;
                    sv[sb][r] = tok < t1 ? x : -INFINITY;
                    bm = fmaxf(bm, sv[sb][r]);
                }
            }
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            const float mn = fmaxf(m, bm);
            const float mref = mn == -INFINITY ? 0.f : mn;
            const float alpha = fast_exp2(m - mref);
            m = mn;
            bf16x8 pb;
            float ps = 0.f;
#pragma unroll
            for (int sb = 0; sb < 2; sb++) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float p = fast_exp2(sv[sb][r] - mref);
                    if (FP8) {
                        ps += p;
                        pb[4 * sb + r] = (__bf16)(p * cur.vs[sb]);
                    } else {
                        const __bf16 pr = (__bf16)p;
                        ps += (float)pr;
                        pb[4 * sb + r] = pr;
                    }
                }
            }
            l = l * alpha + ps;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int i = 0; i < C::NDB; i++) acc[i] *= alpha;
            }

            // ---- O^T += V^T . P^T  (V^T rows come back transposed from the LDS tile)
#pragma unroll
            for (int db = 0; db < C::NDB; db++) {
                bf16x8 va;
                if (FP8) {
                    const int jj = lane & 15;
                    const int rr = jj >> 1;                            // operand row = k index
                    const int tok = rr < 4 ? 4 * g4 + rr : 16 + 4 * g4 + (rr - 4);
                    const uint8_t *p = vt + tok * C::RS + 16 * db + 8 * (jj & 1);
                    i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2 *)(
                            (__attribute__((address_space(3))) uint8_t *)p));
                    va = e4m3x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]);
                } else {
                    const int jj = lane & 15;
                    const int rr = jj >> 2;
                    bf16x4 lo, hi;
                    {
                        const uint8_t *p = vt + (4 * g4 + rr) * C::RS + (16 * db + 4 * (jj & 3)) * 2;
                        lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (__attribute__((address_space(3))) bf16x4 *)(
                                (__attribute__((address_space(3))) uint8_t *)p));
                    }
                    {
                        const uint8_t *p = vt + (16 + 4 * g4 + rr) * C::RS + (16 * db + 4 * (jj & 3)) * 2;
                        hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (__attribute__((address_space(3))) bf16x4 *)(
                                (__attribute__((address_space(3))) uint8_t *)p));
                    }
                    va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
                    va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
                }
                acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[db], 0, 0, 0);
            }
            cur = nxt;
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

        // ---- write: 8 consecutive dims of one head per thread
        {
            const int t = threadIdx.x;
            const int head = t / (D / 8), d0 = (t % (D / 8)) * 8;
            if (head < G && t < 16 * (D / 8)) {
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
                const int64_t row = (int64_t)b * Hq + (int64_t)h * G + head;
                if (flags & 1) {
                    bf16x8 ob;
#pragma unroll
                    for (int k = 0; k < 8; k++) ob[k] = (__bf16)o[k];
                    *(bf16x8 *)(a.out + row * a.Dv + d0) = ob;
                    if (d0 == 0) a.lse[row] = lse_v;
                } else {
                    const int64_t prow = ((int64_t)it * a.Hkv + h) * G + head;
                    float *dst = a.ws_o + prow * a.Dv + d0;
                    *(f32x4 *)dst = f32x4{o[0], o[1], o[2], o[3]};
                    *(f32x4 *)(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
                    if (d0 == 0) a.ws_lse[prow] = lse_v;
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    const dim3 grid(a.num_parts, a.Hkv), block(kThreads);
    const bool fp8 = a.kv_format == PA_KV_FP8_E4M3_PAGE_HEAD;
    if (a.D == 128 && !fp8)
        hipLaunchKernelGGL((pa_decode_kernel<128, false>), grid, block, 0, stream, a);
    else if (a.D == 64 && !fp8)
        hipLaunchKernelGGL((pa_decode_kernel<64, false>), grid, block, 0, stream, a);
    else if (a.D == 128 && fp8)
        hipLaunchKernelGGL((pa_decode_kernel<128, true>), grid, block, 0, stream, a);
    else if (a.D == 64 && fp8)
        hipLaunchKernelGGL((pa_decode_kernel<64, true>), grid, block, 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
