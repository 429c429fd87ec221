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
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_swap2(float v) {  // lane ^ 2 within a quad
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
}
// The workgroup is a single wave and LDS operations of a wave complete in
// order, so ordering LDS writes before other lanes' reads needs only a
// wave-scope fence; a workgroup barrier would also wait for the next page's
// global loads that are in flight and defeat the prefetch.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, 64); }

// Cross-lane steps on the VALU (no LDS round trip).  permlane16/32_swap of a
// value with itself returns, in every lane l, the values of lanes l and
// l ^ 16 (resp. l ^ 32) of the pair.
__device__ __forceinline__ float xmax16(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int CTRL>
__device__ __forceinline__ float dppc(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// max over the whole wave, in every lane
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dppc<0x128>(v));  // row_ror:8
    v = fmaxf(v, dppc<0x124>(v));  // row_ror:4
    v = fmaxf(v, dppc<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dppc<0xB1>(v));   // quad_perm [1,0,3,2]
    return xmax32(xmax16(v));
}
// every lane gets the value of lane (l % 16) of the first row
__device__ __forceinline__ float bcast_row0(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    auto b = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
    return __uint_as_float(b[0]);
}
// lane (r, G4) gets the value of lane 4 G4 (a per-row broadcast from row 0)
__device__ __forceinline__ float from_lane4g(float v, int G4) {
    float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 4));
    float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 8));
    float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 12));
    return G4 == 0 ? a0 : G4 == 1 ? a1 : G4 == 2 ? a2 : a3;
}
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

// Page loads go through a buffer descriptor of the page itself: 32-bit lane
// offsets (constant parts folded into the instruction), no 64-bit address
// arithmetic, and any offset past the page reads zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t *pg, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(pg), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ void load_meta(PageRegs &R, __amdgpu_buffer_rsrc_t rs,
                                          const PageLayout &Ly, int lane, int meta_chunks,
                                          uint32_t meta_a_bytes) {
    // metadata: [K_scale K_zero K_idx] then [V_scale V_zero]
#pragma unroll
    for (int i = 0; i < 5; i++) {
        int ch = min(lane + 64 * i, meta_chunks - 1);
        uint32_t off = 16u * ch;
        off = off < meta_a_bytes ? Ly.ks + off : Ly.vs + (off - meta_a_bytes);
        u4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
        R.meta[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

template <int KH>
__device__ __forceinline__ void load_codes(PageRegs &R, __amdgpu_buffer_rsrc_t rs,
                                           const PageLayout &Ly, int k, int lane) {
    const int r = lane & 15, G4 = lane >> 4;
    // Every load is issued unconditionally (indices clamped into the page) so
    // the number of loads in flight is static and the compiler can wait for
    // the current page's data without draining the prefetch of the next.
    const int klo_off = (int)Ly.klo + r * 32 + 8 * G4;
#pragma unroll
    for (int mt = 0; mt < 8; mt++) {
        auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, klo_off + 512 * mt, 0, 0);
        R.klo[mt] = make_uint2(v[0], v[1]);
    }
#pragma unroll
    for (int mt = 0; mt < 8; mt++) {
#pragma unroll
        for (int ms = 0; ms < KH; ms++) {
            int dw = 2 * ms + (G4 >> 1);
            int dwc = dw < k / 16 ? dw : k / 16 - 1;
            uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(
                rs, (int)Ly.khi + (16 * mt + r) * (k / 4) + 4 * dwc, 0, 0);
            R.khi[mt][ms] = dw < k / 16 ? v : 0u;
        }
    }
#pragma unroll
    for (int s = 0; s < 4; s++) {
        u4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)Ly.vc + 16 * lane + 1024 * s, 0, 0);
        R.vc[s] = make_uint4(v[0], v[1], v[2], v[3]);
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
    __shared__ __align__(16) uint8_t meta[5 * 64 * 16];  // page metadata copy (16-byte chunks)
    __shared__ __align__(16) u4_t wB[HQ][2][64];                     // lo-plane weights [hi/lo][lane]
    __shared__ __align__(16) u4_t wBh[HQ][4][KH > 0 ? KH : 1][2][16];  // hi-plane weights [group]
    __shared__ __align__(16) float vsf[D / GV][144];                   // V scale x 2^Eu, padded rows
    __shared__ __align__(16) u4_t tq3[HQ][4][64];   // q pieces: B operand of the zero-point MFMA
    __shared__ __align__(16) float tqs[HQ][64][8];  // q / 4^sig of each producer lane's slots
    __shared__ __align__(16) float vzf[D / GV][144];                   // V zero, padded rows
    __shared__ float sw[G][32];

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int unit = b * Hkv + h;
    const int Hq = Hkv * G;
    const int lane = threadIdx.x, r = lane & 15, G4 = lane >> 4;

    // q of the G query heads: one 16-byte load per lane per 64 chunks of 8 channels
    for (int ch = lane; ch < G * (D / 8); ch += 64) {
        int hh = ch / (D / 8), c0 = 8 * (ch % (D / 8));
        uint4 v = *reinterpret_cast<const uint4 *>(q + ((size_t)b * Hq + h * G + hh) * D + c0);
        uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; e++)
            qf[hh][c0 + e] = dec<DT>((uint16_t)(wv[e >> 1] >> (16 * (e & 1)))) * qscale;
    }
    wave_sync();

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
            float p = tl < nt ? __builtin_amdgcn_exp2f(s[j] - mx) : 0.0f;
            float l = p;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) l += shfl_xor(l, o);
            mrow[j] = mx;
            lrow[j] = l;
            int hh = hs + 2 * j;
            if (hh < G) sw[hh][tl] = p;
        }
        wave_sync();
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
    // (column 4 h' + piece, pieces 0..2; k slot 8 G4 + e <-> channel 32 m + 8 G4 + e).
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
            tq3[qd][m][lane] = u4_t{dw[0], dw[1], dw[2], dw[3]};
        }
    }
    // Weight producer role of this lane (lo plane): K step pm = lane / 16, lane
    // group pG = (lane / 4) % 4 and head ph = lane % 4 of each quad; its eight
    // channels are pbase + i + 8 e (i < 4, e < 2), k slots 8 pG + 2 i + e of
    // MFMA pm.  The 16 bytes it writes per (quad, hi/lo) are exactly what
    // reader lane (col 4 ph + hi/lo, pG) loads for MFMA pm.
    const int pm = lane >> 4, pG = (lane >> 2) & 3, ph = lane & 3;
    const int pbase = 32 * pG + 16 * (pm >> 1) + 4 * (pm & 1);
#pragma unroll
    for (int qd = 0; qd < HQ; qd++)  // q'(head, channel) / 4^sig of this lane's slots
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int e = 0; e < 2; e++) {
                int hh = 4 * qd + ph;
                float sig = 1.0f / (float)(1 << (2 * code_sig(4 * (pm & 1) + i)));
                tqs[qd][lane][2 * i + e] = hh < G ? qf[hh][pbase + i + 8 * e] * sig : 0.0f;
            }
    // hi-plane producer role: lane group hG and head ph (group = lane / 16)
    const int hG = (lane >> 2) & 3;
    const int hjb = 16 * (hG >> 1) + 4 * (hG & 1);
    float qmax = 0.0f;
    for (int i = lane; i < G * D; i += 64) qmax = fmaxf(qmax, fabsf(qf[i / D][i % D]));
    qmax = wave_max(qmax);

    float acc[HQ][8];  // lane (r, G4): head 4 qd + G4, channel 16 n + r (scaled by 2^Eu ...)
    float m_run[HQ], l_part[HQ], zt[HQ];
#pragma unroll
    for (int qd = 0; qd < HQ; qd++) {
        m_run[qd] = -INFINITY;
        l_part[qd] = 0.0f;
        zt[qd] = 0.0f;
#pragma unroll
        for (int n = 0; n < 8; n++) acc[qd][n] = 0.0f;
    }
    int Eu = 1000;

    const int p0 = split * pps;
    const int p1 = min(n_pages, p0 + pps);
    const uint8_t *ubase = cache + (size_t)unit * max_pages * page_bytes;
    PageRegs cur;
    {
        const __amdgpu_buffer_rsrc_t rs0 = page_rsrc(ubase + (size_t)p0 * page_bytes, page_bytes);
        load_codes<KH>(cur, rs0, Ly, k, lane);
        load_meta(cur, rs0, Ly, lane, meta_chunks, meta_a);
    }

    for (int p = p0; p < p1; p++) {
        // prefetch of the next page (the last page is loaded again at the end:
        // harmless): codes now, metadata once this page's copy is in LDS
        const __amdgpu_buffer_rsrc_t rsn =
            page_rsrc(ubase + (size_t)min(p + 1, p1 - 1) * page_bytes, page_bytes);
        PageRegs nxt;
        load_codes<KH>(nxt, rsn, Ly, k, lane);
        wave_sync();  // previous page's LDS reads are done
#pragma unroll
        for (int i = 0; i < 5; i++) reinterpret_cast<uint4 *>(meta)[lane + 64 * i] = cur.meta[i];
        load_meta(nxt, rsn, Ly, lane, meta_chunks, meta_a);

        // Page exponent of the weights: |4 w 2^E / 4^sig| <= qmax max(s) 2^(E-2) <= 2^14.
        float smax = 0.0f;
        {
            uint4 c = cur.meta[0];  // chunks 0..63 are exactly K_scale (1024 B)
            uint32_t wv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 8; e++)
                smax = fmaxf(smax, fabsf(dec<DT>((uint16_t)(wv[e >> 1] >> (16 * (e & 1))))));
            smax = wave_max(smax);
        }
        int eb;
        frexpf(qmax * smax, &eb);
        const int E = __builtin_amdgcn_readfirstlane(min(100, max(-60, 16 - eb)));
        const float wscale = ldexpf(1.0f, E);
        const float sback = ldexpf(1.0f, 24 - E);
        wave_sync();

        // Value scales and zeros as fp32 tables (padded rows: conflict-free reads),
        // scales multiplied by 2^Eu so that u = p s_v splits into normal fp16 parts.
        float vsr[8], vzr[8];
        {
            const int cg = lane >> 4, t8 = 8 * (lane & 15);
            uint4 sv = *reinterpret_cast<const uint4 *>(mvs + cg * P + t8);
            uint4 zv = *reinterpret_cast<const uint4 *>(mvz + cg * P + t8);
            uint32_t sw4[4] = {sv.x, sv.y, sv.z, sv.w}, zw4[4] = {zv.x, zv.y, zv.z, zv.w};
            float vmax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                vsr[e] = dec<DT>((uint16_t)(sw4[e >> 1] >> (16 * (e & 1))));
                vzr[e] = dec<DT>((uint16_t)(zw4[e >> 1] >> (16 * (e & 1))));
                vmax = fmaxf(vmax, fabsf(vsr[e]));
            }
            vmax = wave_max(vmax);
            int ev;
            frexpf(vmax, &ev);
            const int Eu_new = __builtin_amdgcn_readfirstlane(min(Eu, min(100, max(-60, 14 - ev))));
            const float urescale = ldexpf(1.0f, max(Eu_new - Eu, -126));
            Eu = Eu_new;
            const float uscale = ldexpf(1.0f, Eu);
#pragma unroll
            for (int e = 0; e < 8; e++) vsr[e] *= uscale;
            float *vst = &vsf[cg][t8];
            float *vzt = &vzf[cg][t8];
            *reinterpret_cast<float4 *>(vst) = make_float4(vsr[0], vsr[1], vsr[2], vsr[3]);
            *reinterpret_cast<float4 *>(vst + 4) = make_float4(vsr[4], vsr[5], vsr[6], vsr[7]);
            *reinterpret_cast<float4 *>(vzt) = make_float4(vzr[0], vzr[1], vzr[2], vzr[3]);
            *reinterpret_cast<float4 *>(vzt + 4) = make_float4(vzr[4], vzr[5], vzr[6], vzr[7]);
#pragma unroll
            for (int qd = 0; qd < HQ; qd++)
#pragma unroll
                for (int n = 0; n < 8; n++) acc[qd][n] *= urescale;
        }

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
                for (int m = 0; m < 4; m++) cb = mfma_dt<DT>(az[m], tq3[qd][m][lane], cb);
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    float v = cb[g];
                    v += dpp_quad_swap1(v);
                    v += dpp_quad_swap2(v);
                    bias[qd][g] = bcast_row0(v);  // rows 0..3 live in lanes 0..15
                }
            }
        }
        // Hi-plane weights of all four groups, once per page: lane = 16 g + 4 hG + ph
        // computes 4 q'(head, idx[j]) s(g, idx[j]) 2^E / 4^sig_hi(i) for the boosted
        // slots j = 32 ms + 16 (hG / 2) + 4 (hG % 2) + i + 8 e of K step ms.
#pragma unroll
        for (int ms = 0; ms < KH; ms++) {
            const int hg = lane >> 4;
            float wv[HQ][4][2];
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int e = 0; e < 2; e++) {
                    const int j = 32 * ms + hjb + i + 8 * e;
                    const int c = j < k ? (int)midx[j] : -1;
                    const float sv = c >= 0 ? dec<DT>(mks[hg * D + c]) : 0.0f;
                    const float f = 4.0f * wscale / (float)(1 << (2 * (2 + (i & 1))));
#pragma unroll
                    for (int qd = 0; qd < HQ; qd++) {
                        const int hh = 4 * qd + ph;
                        wv[qd][i][e] = c >= 0 && hh < G ? qf[hh][c] * sv * f : 0.0f;
                    }
                }
#pragma unroll
            for (int qd = 0; qd < HQ; qd++) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; i++) split2(wv[qd][i][0], wv[qd][i][1], hi[i], lo[i]);
                wBh[qd][hg][ms][0][lane & 15] = u4_t{hi[0], hi[1], hi[2], hi[3]};
                wBh[qd][hg][ms][1][lane & 15] = u4_t{lo[0], lo[1], lo[2], lo[3]};
            }
        }
        float qlo[HQ][4][2];
#pragma unroll
        for (int qd = 0; qd < HQ; qd++) {
            float4 a = *reinterpret_cast<const float4 *>(&tqs[qd][lane][0]);
            float4 c = *reinterpret_cast<const float4 *>(&tqs[qd][lane][4]);
            const float t8[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int e = 0; e < 2; e++) qlo[qd][i][e] = t8[2 * i + e] * wscale;
        }

        const int cgr = r & 3;  // Value group of this lane's PV row
#pragma unroll
        for (int g = 0; g < 4; g++) {
            // --- weights of this group into LDS: lo plane and hi plane ---
            wave_sync();  // previous group's weight reads are done
            {
                uint2 sa = *reinterpret_cast<const uint2 *>(mks + g * D + pbase);
                uint2 sb = *reinterpret_cast<const uint2 *>(mks + g * D + pbase + 8);
                float s0[4] = {dec<DT>((uint16_t)(sa.x & 0xffff)), dec<DT>((uint16_t)(sa.x >> 16)),
                               dec<DT>((uint16_t)(sa.y & 0xffff)), dec<DT>((uint16_t)(sa.y >> 16))};
                float s1[4] = {dec<DT>((uint16_t)(sb.x & 0xffff)), dec<DT>((uint16_t)(sb.x >> 16)),
                               dec<DT>((uint16_t)(sb.y & 0xffff)), dec<DT>((uint16_t)(sb.y >> 16))};
#pragma unroll
                for (int qd = 0; qd < HQ; qd++) {
                    uint32_t hi[4], lo[4];
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        split2(qlo[qd][i][0] * s0[i], qlo[qd][i][1] * s1[i], hi[i], lo[i]);
                    wB[qd][0][lane] = u4_t{hi[0], hi[1], hi[2], hi[3]};
                    wB[qd][1][lane] = u4_t{lo[0], lo[1], lo[2], lo[3]};
                }
            }
            wave_sync();
#pragma unroll
            for (int qd = 0; qd < HQ; qd++) {
                // --- QK on the matrix cores: two 16-token tiles ---
                const int hl = r & 1, hp = r >> 2;
                u4_t bw[4 + (KH > 0 ? KH : 1)];
#pragma unroll
                for (int m = 0; m < 4; m++) bw[m] = wB[qd][hl][16 * m + 4 * G4 + hp];
#pragma unroll
                for (int ms = 0; ms < KH; ms++) bw[4 + ms] = wBh[qd][g][ms][hl][4 * G4 + hp];
                float sc[2][4];
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
                    for (int e = 0; e < 4; e++)
                        sc[mt][e] = fmaf(c[e] + dpp_quad_swap1(c[e]), sback, bias[qd][g]);
                }

                // --- online softmax over these 32 tokens, per head ---
                float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                                 fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
                mx = xmax32(xmax16(mx));
                if (__any(mx > m_run[qd])) {  // wave-uniform: rescale only when a max grows
                    float mnew = fmaxf(m_run[qd], mx);
                    float alpha = __builtin_amdgcn_exp2f(m_run[qd] - mnew);
                    m_run[qd] = mnew;
                    l_part[qd] *= alpha;
                    zt[qd] *= alpha;
                    // accumulator lanes hold head G4 of the quad: that head's alpha
                    float al = from_lane4g(alpha, G4);
#pragma unroll
                    for (int n = 0; n < 8; n++) acc[qd][n] *= al;
                }
                float pr[2][4];
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        pr[mt][e] = __builtin_amdgcn_exp2f(sc[mt][e] - m_run[qd]);
                        l_part[qd] += pr[mt][e];
                    }

                // --- PV on the matrix cores (32 tokens x 16-channel tiles) ---
                uint32_t ahi[4], alo[4];
                {
                    const int t = 32 * g + 4 * G4;
                    float4 s0 = *reinterpret_cast<const float4 *>(&vsf[cgr][t]);
                    float4 s1 = *reinterpret_cast<const float4 *>(&vsf[cgr][t + 16]);
                    float4 z0 = *reinterpret_cast<const float4 *>(&vzf[cgr][t]);
                    float4 z1 = *reinterpret_cast<const float4 *>(&vzf[cgr][t + 16]);
                    const float vs8[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                    const float vz8[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
                    for (int e2 = 0; e2 < 4; e2++) {
                        float pa = pr[e2 >> 1][2 * (e2 & 1)], pb = pr[e2 >> 1][2 * (e2 & 1) + 1];
                        split2(pa * vs8[2 * e2], pb * vs8[2 * e2 + 1], ahi[e2], alo[e2]);
                        zt[qd] = fmaf(pa, vz8[2 * e2], fmaf(pb, vz8[2 * e2 + 1], zt[qd]));
                    }
                }
                const u4_t a_hi = {ahi[0], ahi[1], ahi[2], ahi[3]};
                const u4_t a_lo = {alo[0], alo[1], alo[2], alo[3]};
                const uint4 vb = cur.vc[g];
                const Codes8 v0(vb.x), v1(vb.y), v2(vb.z), v3(vb.w);
#pragma unroll
                for (int n = 0; n < 8; n++) {
                    const u4_t bv = {v0[n], v1[n], v2[n], v3[n]};
                    f4_t cs = mfma_f16(a_hi, bv, f4_t{0, 0, 0, 0});
                    cs = mfma_f16(a_lo, bv, cs);
                    acc[qd][n] += cs[n >> 1];
                }
            }
        }
        cur = nxt;
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
        float w = __builtin_amdgcn_exp2f(ws_ml[(bq * max_splits + s) * 2] - M);
        num = fmaf(w, ws_acc[(bq * max_splits + s) * D + c], num);
        den = fmaf(w, ws_ml[(bq * max_splits + s) * 2 + 1], den);
    }
    out[bq * D + c] = num / den;
}

// Resident workgroups of this instantiation on the whole device (occupancy API),
// cached; 2048 when no device answers (host-only use).
template <int DT, int G, int KH>
int slots3() {
    static int cached = 0;
    if (cached) return cached;
    int per_cu = 0, dev = 0;
    hipDeviceProp_t prop;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<DT, G, KH>,
                                                     64, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        per_cu <= 0) {
        (void)hipGetLastError();
        return 2048;
    }
    cached = per_cu * prop.multiProcessorCount;
    return cached;
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

template <int DT, int G>
int slots2(int k) {
    switch ((k + 31) / 32) {
        case 0: return slots3<DT, G, 0>();
        case 1: return slots3<DT, G, 1>();
        case 2: return slots3<DT, G, 2>();
        case 3: return slots3<DT, G, 3>();
        default: return slots3<DT, G, 4>();
    }
}
template <int DT>
int slots1(int g, int k) {
    switch (g) {
        case 1: return slots2<DT, 1>(k);
        case 2: return slots2<DT, 2>(k);
        case 4: return slots2<DT, 4>(k);
        case 8: return slots2<DT, 8>(k);
        default: return slots2<DT, 16>(k);
    }
}

}  // namespace

int decode_slots(const Geometry &G) {
    return G.dtype == F16 ? slots1<F16>(G.g, G.k) : slots1<BF16>(G.g, G.k);
}

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
