// kvq_decode.hip -- split-K GQA decode attention over the packed cache (gfx950).
//
// Grid (split, KV head, sequence); one 64-lane wave per workgroup.  A page
// split streams its pages with 128-bit loads (the next page is in flight
// while the current one is computed) and contracts them on the matrix cores:
//
//  QK  (16 tokens x 32 channels) x (32 channels x 16 columns) per MFMA.  The
//      A operand is the 2-bit Key code itself: masking a packed word (or the
//      word shifted by 4 or -6) leaves two codes at mantissa bits 4..9 of two
//      fp16 halves, i.e. the exact subnormals code * 4^sig * 2^-24 with sig in
//      {2, 3, 4}, so unpacking costs about one instruction per two codes.  (The
//      matrix cores keep full precision for such operands only when the code
//      sits at bit 4 or above: at bits 0..3 low-order product bits are lost.)
//      The B operand holds the per-group weights w = q * scale * log2(e) * s
//      (Key scale of the channel and 32-token group) * 2^E / 4^sig, split
//      into an fp16 hi and lo part in neighbouring columns so that the
//      products keep ~22 bits.  Boosted channels (Kitty
//      abstract: two uniform 2-bit planes per mixed-precision Key page) add a
//      second contraction of the hi plane against 4 w of the listed channels.
//      The zero-point term q . z per group comes from one small MFMA of the
//      page's Key zeros against q split into three pieces.
//  PV  (16 rows = 4 heads x 4 Value groups) x (32 tokens x 16 channels): the
//      A operand is p * s_v (softmax weight times the token's Value scale for
//      the group), again split hi/lo; the B operand is the Value code read the
//      same way as the Key codes.  Only the row whose group matches the
//      channel is kept; the zero-point term p . z_v accumulates on the VALU.
//
// Columns of QK are laid out as 4 per query head (hi, lo, hi, lo), so after
// adding neighbours every lane of a head's quad holds that head's scores for
// exactly the tokens its PV operand needs: no transposes or shuffles between
// the two contractions.  An online softmax in the log2 domain keeps (m, l)
// per head (MiniKV summary: unpack fused into the decode matmul; one read of
// a page serves the whole query group, notes.yuuk.io open questions on GQA).
//
// The window split reads the newest n_res exact tokens (KIVI explainer,
// section 3: full-precision residual) on the VALU, 32 tokens per workgroup.
// A combine kernel merges the partials of all splits.
#include <cmath>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ float dec(uint16_t h) {
    if constexpr (DT == F16) {
        return (float)__builtin_bit_cast(_Float16, h);
    } else {
        return __uint_as_float((uint32_t)h << 16);
    }
}
template <int DT>
__device__ __forceinline__ uint16_t enc(float f) {  // round to nearest even
    if constexpr (DT == F16) {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    } else {
        uint32_t u = __float_as_uint(f);
        u += 0x7fffu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
}

__device__ __forceinline__ f4_t mfma_f16(u4_t a, u4_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                  __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
}
template <int DT>
__device__ __forceinline__ f4_t mfma_dt(u4_t a, u4_t b, f4_t c) {
    if constexpr (DT == F16) {
        return mfma_f16(a, b, c);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a),
                                                       __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
    }
}

typedef float f2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
// fp16 pair of (a, b), round to nearest even (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2_t));
}
__device__ __forceinline__ float lo_half(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_half(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// hi = fp16(x), lo = fp16(x - hi), both rounded to nearest even: x = hi + lo
// to within 2^-22 |x| with an unbiased error (x - hi is exact in fp32).
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pack_rne(a, b);
    lo = pack_rne(a - lo_half(hi), b - hi_half(hi));
}

__device__ __forceinline__ float dpp_quad_swap1(float v) {  // lane ^ 1 within a quad
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_swap2(float v) {  // lane ^ 2 within a quad
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, 64); }
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Code extraction: word x holds 16 two-bit codes, code e of each 16-bit half
// at bits 2e.  Output j (0..7) holds code j of both halves at mantissa bits
// 2 sig(j) (sig in {2, 3, 4}), i.e. fp16 subnormals code * 4^sig * 2^-24:
// codes 0, 1 come from x << 4, codes 2..4 from x, codes 5..7 from x >> 6.
__host__ __device__ constexpr int code_sig(int j) {
    return j == 4 || j == 7 ? 4 : (j == 1 || j == 3 || j == 6) ? 3 : 2;
}
struct Codes8 {
    uint32_t xl, x, xr;
    __device__ __forceinline__ explicit Codes8(uint32_t w) : xl(w << 4), x(w), xr(w >> 6) {}
    __device__ __forceinline__ uint32_t operator[](int j) const {
        uint32_t src = j < 2 ? xl : j < 5 ? x : xr;
        return src & (0x00030003u << (2 * code_sig(j)));
    }
};

struct PageRegs {
    uint2 klo[8];       // K lo plane: token 16 mt + (lane & 15), channels 32 (lane >> 4) + [0, 32)
    uint32_t khi[8][4]; // K hi plane dwords 2 ms + ((lane >> 4) >> 1) of the same tokens
    uint4 vc[4];        // V codes: 16-byte block (step, lane)
    uint4 meta[5];      // metadata copy, 16-byte chunks lane + 64 i
};

template <int KH>
__device__ __forceinline__ void load_page(PageRegs &R, const uint8_t *pg, const PageLayout &Ly,
                                          int k, int lane, int meta_chunks, uint32_t meta_a_bytes) {
    const int r = lane & 15, G4 = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 8; mt++)
        R.klo[mt] = *reinterpret_cast<const uint2 *>(pg + Ly.klo + (16 * mt + r) * 32 + 8 * G4);
#pragma unroll
    for (int mt = 0; mt < 8; mt++) {
#pragma unroll
        for (int ms = 0; ms < KH; ms++) {
            int dw = 2 * ms + (G4 >> 1);
            R.khi[mt][ms] = dw < k / 16
                ? *reinterpret_cast<const uint32_t *>(pg + Ly.khi + (16 * mt + r) * (k / 4) + 4 * dw)
                : 0u;
        }
    }
#pragma unroll
    for (int s = 0; s < 4; s++)
        R.vc[s] = *reinterpret_cast<const uint4 *>(pg + Ly.vc + 1024 * s + 16 * lane);
    // metadata: [K_scale K_zero K_idx] then [V_scale V_zero]
#pragma unroll
    for (int i = 0; i < 5; i++) {
        int ch = lane + 64 * i;
        if (ch < meta_chunks) {
            uint32_t off = 16u * ch;
            off = off < meta_a_bytes ? Ly.ks + off : Ly.vs + (off - meta_a_bytes);
            R.meta[i] = *reinterpret_cast<const uint4 *>(pg + off);
        } else {
            R.meta[i] = make_uint4(0, 0, 0, 0);
        }
    }
}

template <int DT, int G, int KH>
__global__ __launch_bounds__(64) void decode_split_kernel(
    const uint8_t *__restrict__ cache, const uint16_t *__restrict__ q, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int Hkv, int max_pages, uint32_t page_bytes, int k,
    size_t res_base, int n_pages, int n_res, int page_splits, int pps, int max_splits,
    float qscale) {
    constexpr int HQ = (G + 3) / 4;       // quads of query heads
    constexpr int NHW = (G + 1) / 2;      // heads per lane in the window path
    __shared__ float qf[G][D];            // q * scale * log2(e)
    __shared__ __align__(16) uint8_t meta[(P / GK) * D * 4 + 128 + (D / GV) * P * 4];
    __shared__ __align__(16) uint32_t wB[HQ][4 + (KH > 0 ? KH : 1)][4][4][2][4];
    __shared__ float sw[G][32];

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int unit = b * Hkv + h;
    const int Hq = Hkv * G;
    const int lane = threadIdx.x, r = lane & 15, G4 = lane >> 4;

    for (int i = lane; i < G * D; i += 64) {
        int hh = i / D, c = i % D;
        qf[hh][c] = dec<DT>(q[((size_t)b * Hq + h * G + hh) * D + c]) * qscale;
    }
    __syncthreads();

    if (split >= page_splits) {
        // ---------------- window split: 32 exact tokens on the VALU ----------------
        const int w = split - page_splits;
        const int t0 = 32 * w;
        const int nt = min(32, n_res - t0);
        const uint16_t *kw = reinterpret_cast<const uint16_t *>(cache + res_base +
                                                                (size_t)unit * 2 * R * D * 2);
        const uint16_t *vw = kw + (size_t)R * D;
        const int tl = lane & 31, hs = lane >> 5;
        float s[NHW];
#pragma unroll
        for (int j = 0; j < NHW; j++) s[j] = tl < nt ? 0.0f : -INFINITY;
        if (tl < nt) {
            const uint4 *row = reinterpret_cast<const uint4 *>(kw + (size_t)(t0 + tl) * D);
            for (int c8 = 0; c8 < D / 8; c8++) {
                uint4 v = row[c8];
                uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    float kv = dec<DT>((uint16_t)(wv[e >> 1] >> (16 * (e & 1))));
#pragma unroll
                    for (int j = 0; j < NHW; j++) {
                        int hh = hs + 2 * j;
                        if (hh < G) s[j] = fmaf(qf[hh][8 * c8 + e], kv, s[j]);
                    }
                }
            }
        }
        float mrow[NHW], lrow[NHW];
#pragma unroll
        for (int j = 0; j < NHW; j++) {
            float mx = s[j];
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
            float p = tl < nt ? exp2f(s[j] - mx) : 0.0f;
            float l = p;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) l += shfl_xor(l, o);
            mrow[j] = mx;
            lrow[j] = l;
            int hh = hs + 2 * j;
            if (hh < G) sw[hh][tl] = p;
        }
        __syncthreads();
        float acc[G][2];
#pragma unroll
        for (int hh = 0; hh < G; hh++) acc[hh][0] = acc[hh][1] = 0.0f;
        for (int t = 0; t < nt; t++) {
            uint32_t vv = *reinterpret_cast<const uint32_t *>(vw + (size_t)(t0 + t) * D + 2 * lane);
            float v0 = dec<DT>((uint16_t)(vv & 0xffffu)), v1 = dec<DT>((uint16_t)(vv >> 16));
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
                float p = sw[hh][t];
                acc[hh][0] = fmaf(p, v0, acc[hh][0]);
                acc[hh][1] = fmaf(p, v1, acc[hh][1]);
            }
        }
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            size_t bq = (size_t)b * Hq + h * G + hh;
            *reinterpret_cast<float2 *>(&ws_acc[(bq * max_splits + split) * D + 2 * lane]) =
                make_float2(acc[hh][0], acc[hh][1]);
        }
#pragma unroll
        for (int j = 0; j < NHW; j++) {
            int hh = hs + 2 * j;
            if (hh < G && tl == 0) {
                size_t bq = (size_t)b * Hq + h * G + hh;
                ws_ml[(bq * max_splits + split) * 2 + 0] = mrow[j];
                ws_ml[(bq * max_splits + split) * 2 + 1] = lrow[j];
            }
        }
        return;
    }

    // ---------------------------- page split ----------------------------
    const PageLayout Ly = page_layout(k);
    const uint32_t meta_a = (P / GK) * D * 4 + (uint32_t)((k + 15) / 16 * 16);  // K scale, zero, idx
    const int meta_chunks = (int)(meta_a + (D / GV) * P * 4) / 16;
    const uint16_t *mks = reinterpret_cast<const uint16_t *>(meta);            // [4][128]
    const uint16_t *mkz = mks + (P / GK) * D;                                  // [4][128]
    const uint8_t *midx = meta + (P / GK) * D * 4;                             // [k]
    const uint16_t *mvs = reinterpret_cast<const uint16_t *>(meta + meta_a);   // [4][128]
    const uint16_t *mvz = mvs + (D / GV) * P;                                  // [4][128]

    // Fixed per call: q pieces as the B operand of the zero-point MFMA
    // (column 4 h' + piece, pieces 0..2; k slot 8 G4 + e <-> channel 32 m + 8 G4 + e),
    // and q of the two channels this lane produces weights for.
    u4_t bq3[HQ][4];
    float qmax = 0.0f;
#pragma unroll
    for (int qd = 0; qd < HQ; qd++) {
        int hh = 4 * qd + (r >> 2), pc = r & 3;
#pragma unroll
        for (int m = 0; m < 4; m++) {
            uint32_t dw[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; e2++) {
                uint16_t pv[2];
#pragma unroll
                for (int u = 0; u < 2; u++) {
                    float x = hh < G ? qf[hh][32 * m + 8 * G4 + 2 * e2 + u] : 0.0f;
                    uint16_t p0 = enc<DT>(x);
                    float r1 = x - dec<DT>(p0);
                    uint16_t p1 = enc<DT>(r1);
                    float r2 = r1 - dec<DT>(p1);
                    uint16_t p2 = enc<DT>(r2);
                    pv[u] = pc == 0 ? p0 : pc == 1 ? p1 : pc == 2 ? p2 : (uint16_t)0;
                }
                dw[e2] = (uint32_t)pv[0] | ((uint32_t)pv[1] << 16);
            }
            bq3[qd][m] = u4_t{dw[0], dw[1], dw[2], dw[3]};
        }
    }
    // producer channels of this lane: c0 = 16 (lane / 8) + lane % 8 and c0 + 8
    const int pc0 = 16 * (lane >> 3) + (lane & 7);
    const int prem = lane & 7;  // extraction index j of (c0, c0 + 8) within its MFMA
    const int pG4 = pc0 >> 5, pm = 2 * ((pc0 & 31) >> 4) + (prem >> 2), pi = prem & 3;
    const float psig = 1.0f / (float)(1 << (2 * code_sig(prem)));
    float qp0[G], qp1[G];
#pragma unroll
    for (int hh = 0; hh < G; hh++) {
        qp0[hh] = qf[hh][pc0];
        qp1[hh] = qf[hh][pc0 + 8];
    }
    for (int i = lane; i < G * D; i += 64) qmax = fmaxf(qmax, fabsf(qf[i / D][i % D]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) qmax = fmaxf(qmax, shfl_xor(qmax, o));

    // hi-plane weight slots beyond k stay zero
    for (int i = lane; i < (int)(sizeof(wB) / 4); i += 64) (&wB[0][0][0][0][0][0])[i] = 0u;

    // PV accumulators: lane (r, G4) keeps, per quad and 16-channel tile n, the
    // one useful MFMA element (row = head G4, Value group n / 2).  Each 32-token
    // step starts its MFMA chain from zero and is added here in fp32 with
    // round-to-nearest: the matrix cores truncate when adding into a large
    // accumulator, which would bias long chains of non-negative products.
    float acc[HQ][8];
#pragma unroll
    for (int qd = 0; qd < HQ; qd++)
#pragma unroll
        for (int n = 0; n < 8; n++) acc[qd][n] = 0.0f;
    float m_run[HQ], l_part[HQ], zt[HQ];
    // PV operand exponent: u = p s_v is scaled by 2^Eu so that its fp16 hi and
    // lo parts stay normal; Eu only decreases along a split, and the
    // accumulators are rescaled exactly when it does.
    int Eu = 1000;
#pragma unroll
    for (int qd = 0; qd < HQ; qd++) {
        m_run[qd] = -INFINITY;
        l_part[qd] = 0.0f;
        zt[qd] = 0.0f;
    }

    const int p0 = split * pps;
    const int p1 = min(n_pages, p0 + pps);
    const uint8_t *ubase = cache + (size_t)unit * max_pages * page_bytes;
    PageRegs cur;
    load_page<KH>(cur, ubase + (size_t)p0 * page_bytes, Ly, k, lane, meta_chunks, meta_a);

    for (int p = p0; p < p1; p++) {
        PageRegs nxt;
        if (p + 1 < p1)
            load_page<KH>(nxt, ubase + (size_t)(p + 1) * page_bytes, Ly, k, lane, meta_chunks,
                          meta_a);
        __syncthreads();  // previous page's metadata reads are done
#pragma unroll
        for (int i = 0; i < 5; i++) {
            int ch = lane + 64 * i;
            if (ch < meta_chunks) reinterpret_cast<uint4 *>(meta)[ch] = cur.meta[i];
        }
        __syncthreads();

        // Page exponent: every weight operand |4 w 2^E / 4^sig| <= |w| 2^(E-2) <=
        // qmax max(s) 2^(E-2) <= 2^14.
        float smax = 0.0f;
        {
            uint4 c = cur.meta[0];  // chunks 0..63 are exactly K_scale (1024 B)
            uint32_t wv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 8; e++)
                smax = fmaxf(smax, fabsf(dec<DT>((uint16_t)(wv[e >> 1] >> (16 * (e & 1))))));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) smax = fmaxf(smax, shfl_xor(smax, o));
        }
        int eb;
        frexpf(qmax * smax, &eb);
        const int E = min(100, max(-60, 16 - eb));
        float vsmax = 0.0f;
        {
            const uint4 c = *reinterpret_cast<const uint4 *>(mvs + 8 * lane);  // V_scale[4][128]
            uint32_t wv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 8; e++)
                vsmax = fmaxf(vsmax, fabsf(dec<DT>((uint16_t)(wv[e >> 1] >> (16 * (e & 1))))));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) vsmax = fmaxf(vsmax, shfl_xor(vsmax, o));
        }
        int ev;
        frexpf(vsmax, &ev);
        const int Eu_new = min(Eu, min(100, max(-60, 14 - ev)));
        const float urescale = ldexpf(1.0f, max(Eu_new - Eu, -126));
        Eu = Eu_new;
        const float uscale = ldexpf(1.0f, Eu);
        const float wscale = ldexpf(1.0f, E);
        const float sback = ldexpf(1.0f, 24 - E);

        // Zero-point term per (head, group): bias = sum_c q'(h, c) z(g, c).
        float bias[HQ][4];
        {
            u4_t az[4];
#pragma unroll
            for (int m = 0; m < 4; m++)
                az[m] = r < 4 ? *reinterpret_cast<const u4_t *>(mkz + r * D + 32 * m + 8 * G4)
                              : u4_t{0, 0, 0, 0};
#pragma unroll
            for (int qd = 0; qd < HQ; qd++) {
                f4_t cb = {0, 0, 0, 0};
#pragma unroll
                for (int m = 0; m < 4; m++) cb = mfma_dt<DT>(az[m], bq3[qd][m], cb);
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    float v = cb[g];
                    v += dpp_quad_swap1(v);
                    v += dpp_quad_swap2(v);
                    bias[qd][g] = shfl(v, r);  // rows 0..3 live in lanes 0..15
                }
            }
        }

        float sc[HQ][4][2][4];  // scores: [quad][group][M-tile][row] for head 4 qd + r / 4
#pragma unroll
        for (int g = 0; g < 4; g++) {
            // --- produce this group's B operands (weights) into LDS ---
            __syncthreads();
            {
                float s0 = dec<DT>(mks[g * D + pc0]) * wscale * psig;
                float s1 = dec<DT>(mks[g * D + pc0 + 8]) * wscale * psig;
#pragma unroll
                for (int hh = 0; hh < G; hh++) {
                    uint32_t hi, lo;
                    split2(qp0[hh] * s0, qp1[hh] * s1, hi, lo);
                    wB[hh >> 2][pm][pG4][hh & 3][0][pi] = hi;
                    wB[hh >> 2][pm][pG4][hh & 3][1][pi] = lo;
                }
                // hi plane: pairs (j0, j0 + 8) of boosted channels, weight 4 w / 4^i
                const int ntask = G * (KH * 16);
                for (int task = lane; task < ntask; task += 64) {
                    int hh = task / (KH * 16), jj = task % (KH * 16);
                    int ms = jj >> 4, rem = jj & 15;  // rem: 16 (G4b / 2) + 4 (G4b % 2) + i
                    int j0 = 32 * ms + 16 * (rem >> 3) + (rem & 7);
                    if (j0 >= k) continue;
                    int G4b = 2 * (rem >> 3) + ((rem & 7) >> 2), i = rem & 3;
                    float f = 4.0f * wscale / (float)(1 << (2 * (2 + (i & 1))));
                    int ca = midx[j0], cb = j0 + 8 < k ? midx[j0 + 8] : -1;
                    float wa = qf[hh][ca] * dec<DT>(mks[g * D + ca]) * f;
                    float wb = cb >= 0 ? qf[hh][cb] * dec<DT>(mks[g * D + cb]) * f : 0.0f;
                    uint32_t hi, lo;
                    split2(wa, wb, hi, lo);
                    wB[hh >> 2][4 + ms][G4b][hh & 3][0][i] = hi;
                    wB[hh >> 2][4 + ms][G4b][hh & 3][1][i] = lo;
                }
            }
            __syncthreads();
            // --- QK on the matrix cores ---
#pragma unroll
            for (int qd = 0; qd < HQ; qd++) {
                u4_t bw[4 + (KH > 0 ? KH : 1)];
#pragma unroll
                for (int m = 0; m < 4 + KH; m++)
                    bw[m] = *reinterpret_cast<const u4_t *>(&wB[qd][m][G4][r >> 2][r & 1][0]);
#pragma unroll
                for (int mt = 0; mt < 2; mt++) {
                    const uint2 kl = cur.klo[2 * g + mt];
                    f4_t c = {0, 0, 0, 0};
                    const Codes8 c0(kl.x), c1(kl.y);
#pragma unroll
                    for (int m = 0; m < 4; m++) {
                        const Codes8 &cx = m < 2 ? c0 : c1;
                        int jb = 4 * (m & 1);
                        u4_t a = {cx[jb], cx[jb + 1], cx[jb + 2], cx[jb + 3]};
                        c = mfma_f16(a, bw[m], c);
                    }
#pragma unroll
                    for (int ms = 0; ms < KH; ms++) {
                        // boosted columns 4 (G4 & 1) + i and + 8 of dword 2 ms + G4 / 2,
                        // at mantissa bits 2 sig_hi(i), sig_hi = {2, 3, 2, 3}
                        uint32_t x = cur.khi[2 * g + mt][ms] >> (8 * (G4 & 1));
                        uint32_t xl = x << 4;
                        u4_t a = {xl & 0x00300030u, xl & 0x00C000C0u, x & 0x00300030u,
                                  x & 0x00C000C0u};
                        c = mfma_f16(a, bw[4 + ms], c);
                    }
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        float v = c[e];
                        v += dpp_quad_swap1(v);  // hi + lo columns
                        sc[qd][g][mt][e] = fmaf(v, sback, bias[qd][g]);
                    }
                }
            }
        }

        // --- online softmax over the page's 128 tokens, per head ---
        float alpha[HQ];
#pragma unroll
        for (int qd = 0; qd < HQ; qd++) {
            float mx = -INFINITY;
#pragma unroll
            for (int g = 0; g < 4; g++)
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e++) mx = fmaxf(mx, sc[qd][g][mt][e]);
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            float mnew = fmaxf(m_run[qd], mx);
            alpha[qd] = exp2f(m_run[qd] - mnew);
            m_run[qd] = mnew;
            float ls = 0.0f;
#pragma unroll
            for (int g = 0; g < 4; g++)
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        float pv = exp2f(sc[qd][g][mt][e] - mnew);
                        sc[qd][g][mt][e] = pv;
                        ls += pv;
                    }
            l_part[qd] = l_part[qd] * alpha[qd] + ls;
            zt[qd] *= alpha[qd];
            // accumulator lanes hold head G4 of the quad: fetch that head's alpha
            float al = shfl(alpha[qd], 4 * G4) * urescale;
#pragma unroll
            for (int n = 0; n < 8; n++) acc[qd][n] *= al;
        }

        // --- PV on the matrix cores, one 32-token step per Key group ---
        const int cgr = r & 3;  // Value group of this lane's PV row
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const uint4 vb = cur.vc[g];
            const uint32_t vx[4] = {vb.x, vb.y, vb.z, vb.w};
            // token scales and zeros of this row's group, tokens 4 G4 + e and 16 + 4 G4 + e
            float vs[8], vz[8];
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
                const int t = 32 * g + 16 * mt + 4 * G4;
                uint2 sv = *reinterpret_cast<const uint2 *>(mvs + cgr * P + t);
                uint2 zv = *reinterpret_cast<const uint2 *>(mvz + cgr * P + t);
                vs[4 * mt + 0] = dec<DT>((uint16_t)(sv.x & 0xffff)) * uscale;
                vs[4 * mt + 1] = dec<DT>((uint16_t)(sv.x >> 16)) * uscale;
                vs[4 * mt + 2] = dec<DT>((uint16_t)(sv.y & 0xffff)) * uscale;
                vs[4 * mt + 3] = dec<DT>((uint16_t)(sv.y >> 16)) * uscale;
                vz[4 * mt + 0] = dec<DT>((uint16_t)(zv.x & 0xffff));
                vz[4 * mt + 1] = dec<DT>((uint16_t)(zv.x >> 16));
                vz[4 * mt + 2] = dec<DT>((uint16_t)(zv.y & 0xffff));
                vz[4 * mt + 3] = dec<DT>((uint16_t)(zv.y >> 16));
            }
            const Codes8 v0(vx[0]), v1(vx[1]), v2(vx[2]), v3(vx[3]);
            u4_t bv[8];
#pragma unroll
            for (int n = 0; n < 8; n++) bv[n] = u4_t{v0[n], v1[n], v2[n], v3[n]};
#pragma unroll
            for (int qd = 0; qd < HQ; qd++) {
                uint32_t ahi[4], alo[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    float pa = sc[qd][g][e2 >> 1][2 * (e2 & 1)];
                    float pb = sc[qd][g][e2 >> 1][2 * (e2 & 1) + 1];
                    split2(pa * vs[2 * e2], pb * vs[2 * e2 + 1], ahi[e2], alo[e2]);
                    zt[qd] = fmaf(pa, vz[2 * e2], fmaf(pb, vz[2 * e2 + 1], zt[qd]));
                }
                u4_t a_hi = {ahi[0], ahi[1], ahi[2], ahi[3]};
                u4_t a_lo = {alo[0], alo[1], alo[2], alo[3]};
#pragma unroll
                for (int n = 0; n < 8; n++) {
                    f4_t cs = mfma_f16(a_hi, bv[n], f4_t{0, 0, 0, 0});
                    cs = mfma_f16(a_lo, bv[n], cs);
                    acc[qd][n] += cs[n >> 1];
                }
            }
        }
        if (p + 1 < p1) cur = nxt;
    }

    // --- partials: lane (c_local = r, G4) owns head 4 qd + G4, channels 16 n + r ---
#pragma unroll
    for (int qd = 0; qd < HQ; qd++) {
        // l and the Value zero term: sum over the four lane groups G4
        float l = l_part[qd];
        l += shfl_xor(l, 16);
        l += shfl_xor(l, 32);
        float z = zt[qd];
        z += shfl_xor(z, 16);
        z += shfl_xor(z, 32);  // lanes (4 h' + cg, *) hold head h', group cg
        const int hh = 4 * qd + G4;
        float lh = shfl(l, 4 * G4);
        float mh = shfl(m_run[qd], 4 * G4);
        float zg[4];
#pragma unroll
        for (int cg = 0; cg < 4; cg++) zg[cg] = shfl(z, 4 * G4 + cg);
        if (hh < G) {
            size_t bq = (size_t)b * Hq + h * G + hh;
            float *dst = ws_acc + (bq * max_splits + split) * D;
#pragma unroll
            for (int n = 0; n < 8; n++)
                dst[16 * n + r] =
                    acc[qd][n] * ldexpf(1.0f, 24 - 2 * code_sig(n) - Eu) + zg[n >> 1];
            if (r == 0) {
                ws_ml[(bq * max_splits + split) * 2 + 0] = mh;
                ws_ml[(bq * max_splits + split) * 2 + 1] = lh;
            }
        }
    }
}

__global__ __launch_bounds__(D) void combine_kernel(const float *__restrict__ ws_ml,
                                                    const float *__restrict__ ws_acc,
                                                    float *__restrict__ out, int total_splits,
                                                    int max_splits) {
    const size_t bq = blockIdx.x;
    const int c = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < total_splits; s++) M = fmaxf(M, ws_ml[(bq * max_splits + s) * 2]);
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < total_splits; s++) {
        float w = exp2f(ws_ml[(bq * max_splits + s) * 2] - M);
        num = fmaf(w, ws_acc[(bq * max_splits + s) * D + c], num);
        den = fmaf(w, ws_ml[(bq * max_splits + s) * 2 + 1], den);
    }
    out[bq * D + c] = num / den;
}

template <int DT, int G, int KH>
hipError_t launch3(const Geometry &Gm, const uint8_t *cache, const uint16_t *q, float *ml,
                   float *acc, const DecodePlan &pl, hipStream_t st) {
    dim3 grid(pl.total_splits, Gm.Hkv, Gm.B);
    hipLaunchKernelGGL((decode_split_kernel<DT, G, KH>), grid, dim3(64), 0, st, cache, q, ml,
                       acc, Gm.Hkv, Gm.max_pages, Gm.page_bytes, Gm.k, Gm.res_base,
                       pl.n_pages, pl.n_res, pl.page_splits, pl.pages_per_split,
                       pl.max_splits, Gm.scale * kLog2e);
    return hipGetLastError();
}

template <int DT, int G>
hipError_t launch2(const Geometry &Gm, const uint8_t *cache, const uint16_t *q, float *ml,
                   float *acc, const DecodePlan &pl, hipStream_t st) {
    switch ((Gm.k + 31) / 32) {
        case 0: return launch3<DT, G, 0>(Gm, cache, q, ml, acc, pl, st);
        case 1: return launch3<DT, G, 1>(Gm, cache, q, ml, acc, pl, st);
        case 2: return launch3<DT, G, 2>(Gm, cache, q, ml, acc, pl, st);
        case 3: return launch3<DT, G, 3>(Gm, cache, q, ml, acc, pl, st);
        case 4: return launch3<DT, G, 4>(Gm, cache, q, ml, acc, pl, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t launch1(const Geometry &Gm, const uint8_t *cache, const uint16_t *q, float *ml,
                   float *acc, const DecodePlan &pl, hipStream_t st) {
    switch (Gm.g) {
        case 1: return launch2<DT, 1>(Gm, cache, q, ml, acc, pl, st);
        case 2: return launch2<DT, 2>(Gm, cache, q, ml, acc, pl, st);
        case 4: return launch2<DT, 4>(Gm, cache, q, ml, acc, pl, st);
        case 8: return launch2<DT, 8>(Gm, cache, q, ml, acc, pl, st);
        case 16: return launch2<DT, 16>(Gm, cache, q, ml, acc, pl, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t decode_workspace_bytes(const Geometry &G, int max_splits) {
    size_t rows = (size_t)G.B * G.Hq * max_splits;
    return rows * 2 * sizeof(float) + rows * D * sizeof(float);
}

hipError_t launch_decode(const Geometry &G, const uint8_t *cache, const uint16_t *q,
                         float *out, void *workspace, const DecodePlan &pl,
                         hipEvent_t ev_before, hipEvent_t ev_after, hipStream_t st) {
    float *ml = reinterpret_cast<float *>(workspace);
    float *acc = ml + (size_t)G.B * G.Hq * pl.max_splits * 2;
    hipError_t e;
    if (ev_before && (e = hipEventRecord(ev_before, st)) != hipSuccess) return e;
    e = G.dtype == F16 ? launch1<F16>(G, cache, q, ml, acc, pl, st)
                       : launch1<BF16>(G, cache, q, ml, acc, pl, st);
    if (e != hipSuccess) return e;
    if (ev_after && (e = hipEventRecord(ev_after, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3(G.B * G.Hq), dim3(D), 0, st, ml, acc, out,
                       pl.total_splits, pl.max_splits);
    return hipGetLastError();
}

}  // namespace kvq
