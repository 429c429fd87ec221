// kvq_decode_core.h -- device code of the split-K GQA decode attention over
// the packed cache (gfx950), shared by the dense cache and the block pool.
//
// A split of one (sequence, KV head) unit is a workgroup of one wave (block
// pool) or four (dense cache: one per SIMD, their partials merged in LDS);
// the kernels map their 1-D grids onto (unit, split).  Each wave of a page
// split streams its run of 32-token Key groups (two 16-token tiles): while a
// group is computed, the next group's codes and metadata (about 3.2 KB) are
// already in flight in a second register set, so a wave needs few registers
// and four waves share each SIMD.
//
//  QK  (16 rows of weights) x (32 channels x 16 tokens) per MFMA.  The B
//      operand is the 2-bit Key code itself: masking a packed word (or the
//      word shifted by 4 or -6) leaves two codes at mantissa bits 4..9 of two
//      fp16 halves, i.e. the exact subnormals code * 4^sig * 2^-24 with sig in
//      {2, 3, 4}, so unpacking costs about one instruction per two codes.  (The
//      matrix cores keep full precision for such operands only when the code
//      sits at bit 4 or above: at bits 0..3 low-order product bits are lost.)
//      The A operand holds the group's weights w = q * scale * log2(e) * s
//      (Key scale of the channel and group) * 2^E / 4^sig, split into an fp16
//      hi and lo row so that the products keep ~22 bits.  Rows are laid out so
//      that output lane (token, row block) holds hi and lo of its own head:
//      every lane owns distinct (head, token) scores and the softmax does no
//      duplicate work.  Boosted channels (Kitty abstract: two uniform 2-bit
//      planes per mixed-precision Key page) add a contraction of the hi plane
//      against 4 w of the listed channels.  The zero-point term q . z per
//      group and head is a VALU dot product: each lane holds the raw q of
//      eight channels for its row's head and takes four packed two-element
//      dot products with the raw Key zeros (exact products, fp32 sums); a row
//      sum over 16 lanes finishes it.
//  PV  (16 rows = 4 heads x 2 Value groups x fp16 hi/lo) x (32 tokens x 16
//      channels): the A operand is p * s_v (softmax weight times the token's
//      Value scale for the group), its hi and lo parts in separate rows, one
//      operand for groups 0-1 and one for groups 2-3; p reaches that layout
//      through a 512-byte LDS transpose.  The B operand is the Value code read
//      the same way as the Key codes.  One product per 16-channel tile; the
//      two rows of the tile's group (hi, lo) are kept and added; the
//      zero-point term p . z_v accumulates on the VALU.
//
// The softmax runs in the log2 domain with a per-head running maximum; the
// weights carry an extra factor 2^Eu (Eu from the largest Value scale seen)
// so that p * s_v always splits into normal fp16 parts.  Partials store
// (m - Eu, l, acc), which the combine step treats like any other maximum.
// (MiniKV summary: unpack fused into the decode matmul; one read of a page
// serves the whole query group, notes.yuuk.io open questions on GQA.)
//
// The window split reads the newest n_res exact tokens (KIVI explainer,
// section 3: full-precision residual) on the VALU, 32 tokens per workgroup.
// A combine kernel merges the partials of all splits.
#pragma once

#include <cmath>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxCombine = kMaxCombineSplits;  // >= 256 page + 4 window splits

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
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef _Float16 hf2_t __attribute__((ext_vector_type(2)));
// c + a.lo b.lo + a.hi b.hi for two packed dtype pairs (products exact in fp32)
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(hf2_t, a), __builtin_bit_cast(hf2_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2_t, a), __builtin_bit_cast(bf2_t, b), c,
                                                false);
}
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
// sum over the whole wave, in every lane
__device__ __forceinline__ float wave_sum(float v) {
    v += dppc<0x128>(v);
    v += dppc<0x124>(v);
    v += dppc<0x4E>(v);
    v += dppc<0xB1>(v);
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
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

typedef unsigned short us2_t __attribute__((ext_vector_type(2)));

// max / sum over the 16 lanes of a row, in every lane of the row
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dppc<0x128>(v));  // row_ror:8
    v = fmaxf(v, dppc<0x124>(v));  // row_ror:4
    v = fmaxf(v, dppc<0x4E>(v));   // quad_perm [2,3,0,1]
    return fmaxf(v, dppc<0xB1>(v));  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float row_sum(float v) {
    v += dppc<0x128>(v);
    v += dppc<0x124>(v);
    v += dppc<0x4E>(v);
    return v + dppc<0xB1>(v);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    v = max(v, dppu<0x128>(v));
    v = max(v, dppu<0x124>(v));
    v = max(v, dppu<0x4E>(v));
    return max(v, dppu<0xB1>(v));
}
// lane (r, R) gets the value held by row (r / 4) (every lane of a row holds the same)
__device__ __forceinline__ float from_row(float v, int row) {
    float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return row == 0 ? a0 : row == 1 ? a1 : row == 2 ? a2 : a3;
}

// Query head served by slot s of lane row R (rows repeat heads when G < 4).
template <int G>
__device__ __forceinline__ int head_of(int R, int s) {
    return G >= 4 ? 4 * s + R : R % G;
}

// Registers of one 32-token Key group (two 16-token tiles) of a page.
template <int KHE>
struct GroupRegs {
    uint2 klo[2];          // K lo plane, tile mt: token 16 mt + (lane & 15), channels 32 (lane >> 4) + [0, 32)
    uint32_t khi[2][KHE];  // K hi plane dwords 2 ms + (lane >> 5) of the same tokens
    u4_t vc;               // V codes: this lane's 16-byte block of the group
    u4_t meta;             // one 16-byte chunk of the group's metadata
    uint32_t ib[KHE][2];   // indices of this lane's two boosted slots (page data)
};

// Page loads go through a buffer descriptor of the page itself: 32-bit lane
// offsets (constant parts folded into the instruction), no 64-bit address
// arithmetic, and any offset past the page reads zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t *pg, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(pg), (short)0, (int)bytes,
                                             0x00020000);
}

// Byte offsets of this lane's loads inside a page (fixed for the whole split).
template <int KHE>
struct LaneOffs {
    int klo, vc, meta, mstride, khi_tile;
    int khi[KHE];
    int idx[KHE][2];
};

// Group g (0..3) of a page: the part of each offset common to all lanes goes
// into the scalar offset.  Every load is issued unconditionally (offsets
// clamped into the page) so the number of loads in flight is static and the
// compiler can wait for one group's data without draining the loads of the
// next.
template <int KH, int KHE>
__device__ __forceinline__ void load_group(GroupRegs<KHE> &Gr, __amdgpu_buffer_rsrc_t rs,
                                           const LaneOffs<KHE> &O, int g) {
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
        auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, O.klo + 512 * mt, 1024 * g, 0);
        Gr.klo[mt] = make_uint2(v[0], v[1]);
    }
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int ms = 0; ms < KH; ms++)
            Gr.khi[mt][ms] = __builtin_amdgcn_raw_buffer_load_b32(
                rs, O.khi[ms] + mt * O.khi_tile, 2 * g * O.khi_tile, 0);
    Gr.vc = __builtin_amdgcn_raw_buffer_load_b128(rs, O.vc, 1024 * g, 0);
    Gr.meta = __builtin_amdgcn_raw_buffer_load_b128(rs, O.meta + g * O.mstride, 0, 0);
#pragma unroll
    for (int ms = 0; ms < KH; ms++)
#pragma unroll
        for (int t = 0; t < 2; t++) Gr.ib[ms][t] = __builtin_amdgcn_raw_buffer_load_b8(rs, O.idx[ms][t], 0, 0);
}

// Waves per SIMD the register allocation aims at (more registers per wave
// beyond that would spill; at eight heads and up to 32 boosted channels the
// compiler keeps a few values that only the partials need in scratch,
// stored before the group loop and read after it).
constexpr int waves_target(int G, int KH) {
    return G <= 4 ? (KH == 0 || (KH == 1 && G > 1) ? 4 : KH <= 3 ? 3 : 2) : G == 8 ? (KH <= 1 ? 4 : KH <= 3 ? 3 : 1) : 1;
}


// Index swizzle of the lo-plane weight table (16-byte entries): bit 1 is
// flipped by bits 3 and 4, so the eight lanes an LDS access serves at a time
// hit eight different bank groups on both the producing and the MFMA side.
__device__ __forceinline__ int wl_swz(int i) { return i ^ ((((i >> 3) ^ (i >> 4)) & 1) << 1); }

// Bytes of the per-wave LDS region of split_body.
template <int G, int KH>
constexpr int split_lds_bytes() {
    constexpr int HQ = (G + 3) / 4, KHE = KH > 0 ? KH : 1, D_ = 128;
    constexpr int page = G * D_ * 2 + HQ * 4 * 32 * 16 + HQ * KHE * 2 * 16 * 16 + 416 * 4 + D_ * 2 +
                         HQ * 4 * (G >= 8 ? 44 : 48) * 4 - (G >= 8 ? D_ * 2 : 0) +
                         (KH > 0 && G <= 4 ? G * D_ * 4 : 0);
    constexpr int win = G * D_ * 4 + 32 * G * 4;
    return page > win ? page : win;
}

// One split of one (sequence, KV head) unit, computed by a workgroup of NW
// waves: window split when split >= page_splits (wave w of window split j
// takes window tokens [32 (NW j + w), +32)), else wave w takes groups
// [(NW split + w) gps, +gps) of the unit's pages.  With NW > 1 the waves'
// partials (m, l, acc) are merged in LDS and the workgroup writes one
// partial; with NW == 1 the wave writes its own.  With POOL the pages of
// sequence b live at pool blocks table[b * max_pages + page] (block = the
// Hkv pages of one 128-token span), otherwise at unit * max_pages + page of a
// dense array.
template <int DT, int G, int KH, bool POOL, int NW = 1>
__device__ __forceinline__ void split_body(
    const uint8_t *__restrict__ cache, uint8_t *__restrict__ window_w,
    const uint16_t *__restrict__ knew, const uint16_t *__restrict__ vnew, int slot,
    const uint16_t *__restrict__ q, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int Hkv, int max_pages, uint32_t page_bytes, int k,
    size_t res_base, int n_pages, int n_res, int page_splits, int gps, int max_splits,
    float qscale, int unit, int split, const int32_t *__restrict__ table) {
    constexpr int HQ = (G + 3) / 4;    // head slots per row of lanes
    constexpr int NQS = (HQ + 1) / 2;  // QK row sets (two slots each)
    constexpr int KHE = KH > 0 ? KH : 1;
    constexpr int NHW = (G + 1) / 2;   // heads per lane in the window path
    // LDS of the page path
    constexpr int O_Q = 0;                                // u16 [G][D] raw q
    constexpr int O_WL = O_Q + G * D * 2;                 // u4 [HQ][4 m][2 x][4 R][4 kb] lo-plane weights
    constexpr int O_WH = O_WL + HQ * 4 * 32 * 16;         // u32 [HQ][KHE][2 x][4 R][4 kb][4] hi plane
    // f32 [416] K scale 2^E [128] | V scale [4 groups][36] | V zero [4][36]
    // (rows padded to 36: the PV-side reads of four groups hit four banks)
    constexpr int O_ST = O_WH + HQ * KHE * 2 * 16 * 16;
    constexpr int PXR = G >= 8 ? 44 : 48;
    // (with eight or more heads the softmax weights reuse the K zero row,
    // which a group reads before it writes them, and their rows are padded
    // less: the region of four waves then fits four workgroups per CU)
    constexpr int O_KZ = O_ST + 416 * 4;                  // u16 [D] K zero of the group
    constexpr int O_PX = G >= 8 ? O_KZ : O_KZ + D * 2;    // f32 [HQ][4][PXR] softmax weights (rows padded)
    constexpr int O_QF = O_PX + HQ * 4 * PXR * 4;         // f32 [G][D] q' (boosted-channel gathers)
    constexpr int LDSB = split_lds_bytes<G, KH>();
    // fp32 q' table for the boosted-channel gathers: only where the LDS it
    // takes does not cost occupancy (G <= 4); larger groups decode raw q
    constexpr bool QF = KH > 0 && G <= 4;
    static_assert(LDSB >= O_QF + (QF ? G * D * 4 : 0), "page LDS");
    static_assert(NW == 1 || LDSB >= G * (D + 2) * 4, "merge area of a wave");
    __shared__ __align__(16) uint8_t lds_all[NW][LDSB];
    // wave index, wave-uniform (page descriptors derived from it stay scalar)
    const int wv = NW > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
    uint8_t *lds = lds_all[wv];

    const int h = unit % Hkv, b = unit / Hkv;
    const int Hq = Hkv * G;
    const int lane = threadIdx.x & 63, r = lane & 15, kb = lane >> 4;
    const uint16_t *qg = q + ((size_t)b * Hq + h * G) * D;
    // partial of this wave: global memory (NW == 1) or its LDS region, laid
    // out [head][acc 0..127, m, l] (NW > 1), merged below
    float *mine = reinterpret_cast<float *>(lds);
    auto put_acc = [&](int hh, int c, float v) {
        if constexpr (NW == 1) {
            const size_t bq = (size_t)b * Hq + h * G + hh;
            ws_acc[partial_index(bq, max_splits, split) * D + c] = v;
        } else {
            mine[hh * (D + 2) + c] = v;
        }
    };
    auto put_ml = [&](int hh, float m, float l) {
        if constexpr (NW == 1) {
            const size_t bq = (size_t)b * Hq + h * G + hh;
            ws_ml[partial_index(bq, max_splits, split) * 2 + 0] = m;
            ws_ml[partial_index(bq, max_splits, split) * 2 + 1] = l;
        } else {
            mine[hh * (D + 2) + D] = m;
            mine[hh * (D + 2) + D + 1] = l;
        }
    };
    auto merge = [&]() {
        if constexpr (NW > 1) {
            __syncthreads();  // every wave's partial is in its LDS region
            for (int i = threadIdx.x; i < G * D; i += 64 * NW) {
                const int hh = i / D, c = i % D;
                float mw[NW], M = -INFINITY;
#pragma unroll
                for (int w = 0; w < NW; w++) {
                    mw[w] = reinterpret_cast<const float *>(lds_all[w])[hh * (D + 2) + D];
                    M = fmaxf(M, mw[w]);
                }
                float a = 0.0f, l = 0.0f;
                if (M > -INFINITY) {
#pragma unroll
                    for (int w = 0; w < NW; w++) {
                        const float *pw = reinterpret_cast<const float *>(lds_all[w]) + hh * (D + 2);
                        const float f = __builtin_amdgcn_exp2f(mw[w] - M);
                        a = fmaf(f, pw[c], a);
                        l = fmaf(f, pw[D + 1], l);
                    }
                }
                const size_t bq = (size_t)b * Hq + h * G + hh;
                ws_acc[partial_index(bq, max_splits, split) * D + c] = a;
                if (c == 0) {
                    ws_ml[partial_index(bq, max_splits, split) * 2 + 0] = M;
                    ws_ml[partial_index(bq, max_splits, split) * 2 + 1] = l;
                }
            }
        }
    };

    if (split >= page_splits) {
        // ---------------- window split: 32 exact tokens on the VALU ----------------
        // Every global load of the split (the token's K row, the V values of
        // this lane's two channels for all 32 tokens, q) is issued before any
        // arithmetic, so the split pays one memory latency.
        const WaveWork ww = wave_work(split, wv, NW, page_splits, gps, n_pages, n_res);
        const int t0 = ww.t0;
        const int nt = ww.t1 - ww.t0;
        const uint16_t *kw = reinterpret_cast<const uint16_t *>(cache + res_base +
                                                                (size_t)unit * 2 * R * D * 2);
        const uint16_t *vw = kw + (size_t)R * D;
        const int tl = lane & 31, hs = lane >> 5;
        constexpr int QCH = (G * (D / 8) + 63) / 64;
        uint4 qraw[QCH];
#pragma unroll
        for (int i = 0; i < QCH; i++)
            qraw[i] = *reinterpret_cast<const uint4 *>(qg + 8 * min(lane + 64 * i, G * (D / 8) - 1));
        // lane (token tl, half hs) holds channels 64 hs + [0, 64) of its token
        // A fused append hands the newest token (window slot `slot`) in knew /
        // vnew: it is read from there and stored into its slot by this split.
        const uint16_t *kn = knew + (size_t)unit * D, *vn = vnew + (size_t)unit * D;
        uint4 kr[D / 16];
        {
            const int tk = t0 + min(tl, nt - 1);
            const uint4 *row = reinterpret_cast<const uint4 *>(
                (tk == slot ? kn : kw + (size_t)tk * D) + 64 * hs);
#pragma unroll
            for (int c8 = 0; c8 < D / 16; c8++) kr[c8] = row[c8];
        }
        uint32_t vr[32];
#pragma unroll
        for (int t = 0; t < 32; t++) {
            const int tv = t0 + min(t, nt - 1);
            vr[t] = *reinterpret_cast<const uint32_t *>((tv == slot ? vn : vw + (size_t)tv * D) +
                                                        2 * lane);
        }
        if (slot >= t0 && slot < t0 + nt && lane < 32) {
            uint16_t *dst = reinterpret_cast<uint16_t *>(window_w + res_base +
                                                         (size_t)unit * 2 * R * D * 2) +
                            (lane < 16 ? 0 : (size_t)R * D) + (size_t)slot * D + 8 * (lane & 15);
            *reinterpret_cast<uint4 *>(dst) =
                *reinterpret_cast<const uint4 *>((lane < 16 ? kn : vn) + 8 * (lane & 15));
        }

        float(*qf)[D] = reinterpret_cast<float(*)[D]>(lds);
        float(*sw)[G] = reinterpret_cast<float(*)[G]>(lds + G * D * 4);  // [token][head]
#pragma unroll
        for (int i = 0; i < QCH; i++) {
            const int ch = lane + 64 * i;
            const uint32_t wv[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
            if (ch < G * (D / 8)) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    qf[ch / (D / 8)][8 * (ch % (D / 8)) + e] =
                        dec<DT>((uint16_t)(wv[e >> 1] >> (16 * (e & 1)))) * qscale;
            }
        }
        wave_sync();
        float sg[G];
#pragma unroll
        for (int hh = 0; hh < G; hh++) sg[hh] = 0.0f;
#pragma unroll
        for (int c8 = 0; c8 < D / 16; c8++) {
            const uint32_t wv[4] = {kr[c8].x, kr[c8].y, kr[c8].z, kr[c8].w};
            float kv[8];
#pragma unroll
            for (int e = 0; e < 8; e++) kv[e] = dec<DT>((uint16_t)(wv[e >> 1] >> (16 * (e & 1))));
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
                const float4 qa = *reinterpret_cast<const float4 *>(&qf[hh][64 * hs + 8 * c8]);
                const float4 qb = *reinterpret_cast<const float4 *>(&qf[hh][64 * hs + 8 * c8 + 4]);
                const float q8[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
                for (int e = 0; e < 8; e++) sg[hh] = fmaf(q8[e], kv[e], sg[hh]);
            }
        }
        // both halves of a token: add the partial dot products (lanes l, l ^ 32)
        float s[NHW];
#pragma unroll
        for (int j = 0; j < NHW; j++) s[j] = 0.0f;
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(sg[hh]), __float_as_uint(sg[hh]),
                                                       false, false);
            const float tot = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
            if ((hh & 1) == hs) s[hh >> 1] = tot;  // lane half hs keeps heads hs + 2 j
        }
        float mrow[NHW], lrow[NHW];
#pragma unroll
        for (int j = 0; j < NHW; j++) {
            const float sj = tl < nt ? s[j] : -INFINITY;
            float mx = sj;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
            float p = tl < nt ? __builtin_amdgcn_exp2f(sj - mx) : 0.0f;
            float l = p;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) l += shfl_xor(l, o);
            mrow[j] = mx;
            lrow[j] = l;
            const int hh = hs + 2 * j;
            if (hh < G) sw[tl][hh] = p;
        }
        wave_sync();
        float acc[G][2];
#pragma unroll
        for (int hh = 0; hh < G; hh++) acc[hh][0] = acc[hh][1] = 0.0f;
#pragma unroll
        for (int t = 0; t < 32; t++) {
            const float v0 = dec<DT>((uint16_t)(vr[t] & 0xffffu)), v1 = dec<DT>((uint16_t)(vr[t] >> 16));
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
                const float p = sw[t][hh];  // 0 past the last token
                acc[hh][0] = fmaf(p, v0, acc[hh][0]);
                acc[hh][1] = fmaf(p, v1, acc[hh][1]);
            }
        }
        wave_sync();  // this wave's reads of its LDS region are done
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            put_acc(hh, 2 * lane, acc[hh][0]);
            put_acc(hh, 2 * lane + 1, acc[hh][1]);
        }
#pragma unroll
        for (int j = 0; j < NHW; j++) {
            int hh = hs + 2 * j;
            if (hh < G && tl == 0) put_ml(hh, mrow[j], lrow[j]);
        }
        merge();
        return;
    }

    // ---------------------------- page split ----------------------------
    const PageLayout Ly = page_layout(k);
    // hi-plane producer role: k block hkb, row block hR, operand dword hq
    const int hkb = lane >> 4, hR = (lane >> 2) & 3, hq = lane & 3;
    LaneOffs<KHE> O;
    O.klo = (int)Ly.klo + r * 32 + 8 * kb;
    O.vc = (int)Ly.vc + 16 * lane;
    O.meta = lane < 32 ? (int)Ly.ks + 1024 * (lane >> 4) + 16 * (lane & 15)
                       : (int)Ly.vs + 1024 * ((lane - 32) >> 4) + 256 * ((lane >> 2) & 3) +
                             16 * (lane & 3);
    O.mstride = lane < 32 ? 256 : 64;
    O.khi_tile = 4 * k;
#pragma unroll
    for (int ms = 0; ms < KHE; ms++) {
        const int dw = min(2 * ms + (kb >> 1), max(k / 16 - 1, 0));
        O.khi[ms] = (int)Ly.khi + r * (k / 4) + 4 * dw;
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int j = 32 * ms + 16 * (hkb >> 1) + 4 * (hkb & 1) + hq + 8 * t;
            O.idx[ms][t] = (int)Ly.kidx + min(j, max(k - 1, 0));
        }
    }
    // groups [g0, g1) of this unit (four per page), two register sets in turn
    const WaveWork ww = wave_work(split, wv, NW, page_splits, gps, n_pages, n_res);
    const int g0 = ww.g0, g1 = ww.g1;
    const uint8_t *ubase = cache + (size_t)unit * max_pages * page_bytes;
    auto page_ptr = [&](int p) {
        if constexpr (POOL)
            return cache + ((size_t)table[(size_t)b * max_pages + p] * Hkv + h) * page_bytes;
        else
            return ubase + (size_t)p * page_bytes;
    };
    // The prefetch past the split's last group goes through an empty
    // descriptor: every offset is out of range, so it reads zeros without
    // touching memory and the number of loads in flight stays static.
    auto rs_of = [&](int gi) {
        return page_rsrc(page_ptr(min(gi, g1 - 1) >> 2), gi < g1 ? page_bytes : 0u);
    };
    // The first group's loads go out before the query is staged, so their
    // latency overlaps the set-up below.
    GroupRegs<KHE> ga;
    if (g0 < g1) load_group<KH>(ga, rs_of(g0), O, g0 & 3);

    uint16_t *qr = reinterpret_cast<uint16_t *>(lds + O_Q);
    float *st = reinterpret_cast<float *>(lds + O_ST);
    uint16_t *kz = reinterpret_cast<uint16_t *>(lds + O_KZ);
    float *px = reinterpret_cast<float *>(lds + O_PX);

    float *qf = reinterpret_cast<float *>(lds + O_QF);
    for (int ch = lane; ch < G * (D / 8); ch += 64) {
        const uint4 v = *reinterpret_cast<const uint4 *>(qg + 8 * ch);
        *reinterpret_cast<uint4 *>(qr + 8 * ch) = v;
        if constexpr (QF) {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; e++)
                qf[8 * ch + e] = dec<DT>((uint16_t)(w[e >> 1] >> (16 * (e & 1)))) * qscale;
        }
    }
    wave_sync();
    auto qv = [&](int hh, int c) { return dec<DT>(qr[hh * D + c]) * qscale; };

    // max |q'| < 2^eq bounds the weights together with the group's largest Key scale
    float qmax = 0.0f;
    for (int i = lane; i < G * D; i += 64) qmax = fmaxf(qmax, fabsf(dec<DT>(qr[i])));
    qmax = wave_max(qmax) * fabsf(qscale);
    int eq;
    frexpf(qmax, &eq);
    eq = __builtin_amdgcn_readfirstlane(qmax > 0.0f ? max(eq, -100) : -100);

    // Lo-plane weight producer role: K step pm, k block pkb, row block pR; its
    // eight channels are pcb + i + 8 e (i < 4, e < 2), i.e. operand element
    // 2 i + e of MFMA pm for lanes (row 4 pR + *, pkb).
    const int pm = lane >> 4, pkb = (lane >> 2) & 3, pR = lane & 3;
    const int pcb = 32 * pkb + 16 * (pm >> 1) + 4 * (pm & 1);
    float qpp[HQ][8];  // q'(head, channel) / 4^sig of those slots
#pragma unroll
    for (int s = 0; s < HQ; s++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int hh = head_of<G>(pR, s);
            const float sig = (pm & 1) ? 1.0f / (float)(1 << (2 * code_sig(4 + (e >> 1))))
                                       : 1.0f / (float)(1 << (2 * code_sig(e >> 1)));
            qpp[s][e] = qv(hh, pcb + (e >> 1) + 8 * (e & 1)) * sig;
        }
    // raw q pairs of channels 8 r + [0, 8) for the head of row kb: the
    // zero-point term
    // (held in registers for up to four heads; larger groups read them from
    // LDS at each group)
    constexpr bool QZR = G <= 4;
    uint32_t qz[QZR ? HQ : 1][4];
    if constexpr (QZR) {
#pragma unroll
        for (int s = 0; s < HQ; s++) {
            const u4_t v = *reinterpret_cast<const u4_t *>(qr + head_of<G>(kb, s) * D + 8 * r);
#pragma unroll
            for (int i = 0; i < 4; i++) qz[s][i] = v[i];
        }
    }

    // Hi-plane producer role (hkb, hR, hq, defined above): its boosted slots
    // are j0 = 32 ms + 16 (hkb / 2) + 4 (hkb % 2) + hq and j0 + 8, at mantissa
    // bits 2 sig_hi with sig_hi = 2 + (hq & 1).
    const float fh = (hq & 1) ? 4.0f / 64.0f : 4.0f / 16.0f;
    // ... times 0 for slots past the k listed channels (their index bytes are 0)
    float fhs[KHE][2];
#pragma unroll
    for (int ms = 0; ms < KHE; ms++)
#pragma unroll
        for (int t = 0; t < 2; t++)
            fhs[ms][t] = 32 * ms + 16 * (hkb >> 1) + 4 * (hkb & 1) + hq + 8 * t < k ? fh : 0.0f;

    // staging destinations of this lane's metadata chunk
    // (lanes 16..31 hold raw K zeros: their chunk goes to the K zero row,
    // which follows the fp32 tables)
    const int st_o = lane < 16   ? 8 * lane
                     : lane < 32 ? 416 + 4 * (lane - 16)
                                 : 128 + 144 * ((lane - 32) >> 4) + 36 * ((lane >> 2) & 3) + 8 * (lane & 3);
    const bool st_f32 = lane < 16 || lane >= 32;

    float acc[HQ][8];  // lane (r, R): head head_of(R, s), channel 16 n + r
    float m_run[HQ], l_part[HQ], zt[HQ];
#pragma unroll
    for (int s = 0; s < HQ; s++) {
        m_run[s] = -INFINITY;
        l_part[s] = 0.0f;
        zt[s] = 0.0f;
#pragma unroll
        for (int n = 0; n < 8; n++) acc[s][n] = 0.0f;
    }
    int Eu = 30;
    int hc[KHE][2];
    float qh[HQ][KHE][2];

    // Issue priority by phase of the group (s_setprio; among the waves of a
    // SIMD the higher priority issues first, the older wave on a tie): the
    // metadata -> exponent -> weight chain that starts a group and the
    // softmax highest, the QK matrix-core products lowest, the PV operands
    // and products between.  Measured against one flat priority: 1.3-8 %
    // less time for the split kernel on every workload, 14 % with eight query
    // heads per KV head (the softmax at the top came later: a further 0-1 %).
    // The repeated settings before the PV operands, the PV products and at
    // the end are part of what was measured: each also bounds the compiler's
    // instruction schedule, and without them the eight-head case is slower.
    auto process = [&](const GroupRegs<KHE> &Gr) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(2);
        // boosted channels of the group's page: gather their q'
#pragma unroll
        for (int ms = 0; ms < KH; ms++)
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int c = (int)(Gr.ib[ms][t] & 127u);
                hc[ms][t] = c;
#pragma unroll
                for (int s = 0; s < HQ; s++)
                    qh[s][ms][t] = (QF ? qf[head_of<G>(hR, s) * D + c] : qv(head_of<G>(hR, s), c)) *
                                   fhs[ms][t];
            }
        // ---- metadata: exponents from the largest scales (integer max of the
        // bits: scales are never negative), then fp32 copies into LDS ----
        const u4_t M = Gr.meta;
        {
            us2_t a = __builtin_elementwise_max(__builtin_bit_cast(us2_t, M[0]),
                                                __builtin_bit_cast(us2_t, M[1]));
            us2_t c = __builtin_elementwise_max(__builtin_bit_cast(us2_t, M[2]),
                                                __builtin_bit_cast(us2_t, M[3]));
            a = __builtin_elementwise_max(a, c);
            uint32_t mm = row_max_u32(max((uint32_t)a[0], (uint32_t)a[1]));
            const uint32_t sb = (uint32_t)__builtin_amdgcn_readlane((int)mm, 0);   // K scales
            const uint32_t vb = (uint32_t)__builtin_amdgcn_readlane((int)mm, 32);  // V scales
            const int es = DT == BF16 ? (int)(sb >> 7) - 126 : (int)(sb >> 10) - 14;
            const int ev = DT == BF16 ? (int)(vb >> 7) - 126 : (int)(vb >> 10) - 14;
            // |w 2^E / 4^sig| < 2^(eq + es + E - 4) <= 2^12 (x4 on the hi plane)
            const int E = min(100, max(-100, 16 - eq - es));
            const int Eg = min(30, max(-100, 14 - ev));  // p' s_v < 2^14 with p' <= 2^Eu
            const float wscale = __uint_as_float((uint32_t)(E + 127) << 23);
            if (Eg < Eu) {  // wave-uniform: the weights' headroom shrinks
                const float f = __uint_as_float((uint32_t)(max(Eg - Eu, -126) + 127) << 23);
#pragma unroll
                for (int s = 0; s < HQ; s++) {
                    l_part[s] *= f;
                    zt[s] *= f;
#pragma unroll
                    for (int n = 0; n < 8; n++) acc[s][n] *= f;
                }
                Eu = Eg;
            }
            const float fac = lane < 16 ? wscale : 1.0f;
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; e++) f[e] = dec<DT>((uint16_t)(M[e >> 1] >> (16 * (e & 1)))) * fac;
            wave_sync();  // the previous group's reads of these tables are done
            if (st_f32) {
                *reinterpret_cast<float4 *>(st + st_o) = make_float4(f[0], f[1], f[2], f[3]);
                *reinterpret_cast<float4 *>(st + st_o + 4) = make_float4(f[4], f[5], f[6], f[7]);
            } else {
                *reinterpret_cast<u4_t *>(st + st_o) = M;
            }
            wave_sync();
            // sback = 2^(24 - E) undoes 2^E and the 2^-24 of the code operand
            const float sback = __uint_as_float((uint32_t)(151 - E) << 23);

            // ---- lo-plane weights of this group ----
            {
                const float4 sa = *reinterpret_cast<const float4 *>(st + pcb);
                const float4 sc = *reinterpret_cast<const float4 *>(st + pcb + 8);
                const float s0[4] = {sa.x, sa.y, sa.z, sa.w}, s1[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
                for (int s = 0; s < HQ; s++) {
                    uint32_t hi[4], lo[4];
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        split2(qpp[s][2 * i] * s0[i], qpp[s][2 * i + 1] * s1[i], hi[i], lo[i]);
                    u4_t *wl = reinterpret_cast<u4_t *>(lds + O_WL);
                    const int wi = (s * 4 + pm) * 32 + 4 * pR + pkb;
                    wl[wl_swz(wi)] = u4_t{hi[0], hi[1], hi[2], hi[3]};
                    wl[wl_swz(wi + 16)] = u4_t{lo[0], lo[1], lo[2], lo[3]};
                }
            }
            // ---- hi-plane weights of this group ----
#pragma unroll
            for (int ms = 0; ms < KH; ms++) {
                const float s0 = st[hc[ms][0]], s1 = st[hc[ms][1]];
#pragma unroll
                for (int s = 0; s < HQ; s++) {
                    uint32_t hi, lo;
                    split2(qh[s][ms][0] * s0, qh[s][ms][1] * s1, hi, lo);
                    uint32_t *wh = reinterpret_cast<uint32_t *>(lds + O_WH) +
                                   (((s * KHE + ms) * 2) * 16 + 4 * hR + hkb) * 4 + hq;
                    wh[0] = hi;
                    wh[64] = lo;
                }
            }
            // ---- zero-point term per head: q . K zero (pairwise dot products
            // of the raw values, exact products), eight channels per lane ----
            float bias[HQ];
            {
                const u4_t zr = *reinterpret_cast<const u4_t *>(kz + 8 * r);
#pragma unroll
                for (int s = 0; s < HQ; s++) {
                    u4_t qs;
                    if constexpr (QZR)
                        qs = u4_t{qz[s][0], qz[s][1], qz[s][2], qz[s][3]};
                    else
                        qs = *reinterpret_cast<const u4_t *>(qr + head_of<G>(kb, s) * D + 8 * r);
                    float t = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; i++) t = dot2<DT>(qs[i], zr[i], t);
                    bias[s] = row_sum(t) * qscale;
                }
            }
            wave_sync();

            __builtin_amdgcn_s_setprio(0);
            // ---- QK on the matrix cores: rows (slot pair, row block, hi/lo) ----
            const Codes8 a0(Gr.klo[0].x), a1(Gr.klo[0].y), b0(Gr.klo[1].x), b1(Gr.klo[1].y);
#pragma unroll
            for (int qs = 0; qs < NQS; qs++) {
                const int slot = min(2 * qs + ((r >> 1) & 1), HQ - 1);
                const u4_t *wl = reinterpret_cast<const u4_t *>(lds + O_WL) +
                                 wl_swz(slot * 128 + 16 * (r & 1) + 4 * (r >> 2) + kb);
                f4_t c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0};
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const u4_t w = wl[32 * m];
                    const Codes8 &x0 = m < 2 ? a0 : a1;
                    const Codes8 &x1 = m < 2 ? b0 : b1;
                    const int jb = 4 * (m & 1);
                    c0 = mfma_f16(w, u4_t{x0[jb], x0[jb + 1], x0[jb + 2], x0[jb + 3]}, c0);
                    c1 = mfma_f16(w, u4_t{x1[jb], x1[jb + 1], x1[jb + 2], x1[jb + 3]}, c1);
                }
#pragma unroll
                for (int ms = 0; ms < KH; ms++) {
                    const u4_t w = reinterpret_cast<const u4_t *>(lds + O_WH)[
                        ((slot * KHE + ms) * 2 + (r & 1)) * 16 + 4 * (r >> 2) + kb];
                    // boosted slots 4 (kb & 1) + i and + 8 of dword 2 ms + kb / 2,
                    // at mantissa bits 2 sig_hi(i), sig_hi = {2, 3, 2, 3}
#pragma unroll
                    for (int mt = 0; mt < 2; mt++) {
                        const uint32_t x = Gr.khi[mt][ms] >> (8 * (kb & 1));
                        const uint32_t xl = x << 4;
                        const u4_t bh = {xl & 0x00300030u, xl & 0x00C000C0u, x & 0x00300030u,
                                         x & 0x00C000C0u};
                        if (mt == 0) c0 = mfma_f16(w, bh, c0);
                        else c1 = mfma_f16(w, bh, c1);
                    }
                }
                __builtin_amdgcn_s_setprio(2);
                // ---- online softmax: lane (token r, row kb) owns its head's scores ----
#pragma unroll
                for (int a = 0; a < 2; a++) {
                    const int s = 2 * qs + a;
                    if (s >= HQ) break;
                    const float sc0 = fmaf(c0[2 * a] + c0[2 * a + 1], sback, bias[s]);
                    const float sc1 = fmaf(c1[2 * a] + c1[2 * a + 1], sback, bias[s]);
                    const float mx = row_max(fmaxf(sc0, sc1));
                    if (__any(mx > m_run[s])) {  // wave-uniform: rescale only when a max grows
                        const float mnew = fmaxf(m_run[s], mx);
                        const float alpha = __builtin_amdgcn_exp2f(m_run[s] - mnew);
                        m_run[s] = mnew;
                        l_part[s] *= alpha;
#pragma unroll
                        for (int n = 0; n < 8; n++) acc[s][n] *= alpha;
                        zt[s] *= from_row(alpha, r >> 2);  // zt lanes hold head row r / 4
                    }
                    const float mo = m_run[s] - (float)Eu;
                    const float p0 = __builtin_amdgcn_exp2f(sc0 - mo);
                    const float p1 = __builtin_amdgcn_exp2f(sc1 - mo);
                    l_part[s] += p0 + p1;
                    px[(s * 4 + kb) * PXR + r] = p0;
                    px[(s * 4 + kb) * PXR + 16 + r] = p1;
                }
            }
            wave_sync();
        }

        __builtin_amdgcn_s_setprio(1);
        // ---- PV on the matrix cores (32 tokens x 16-channel tiles) ----
        // Rows r = 4 R' + 2 g' + hl of A operand (s, gp) hold part hl (fp16
        // hi or lo) of p' s_v for head slot s of row R' and Value group
        // 2 gp + g'; a tile of group g takes operand g / 2 and keeps its
        // rows g' = g % 2.  Lane pairs (hl = 0, 1) compute one group each
        // (2 hl + g') and swap the parts the other needs.
        u4_t a0[HQ], a1[HQ];
        {
            const int hl = r & 1, gsel = 2 * hl + ((r >> 1) & 1);
            const float4 va = *reinterpret_cast<const float4 *>(st + 128 + 36 * gsel + 4 * kb);
            const float4 vb = *reinterpret_cast<const float4 *>(st + 128 + 36 * gsel + 16 + 4 * kb);
            const float4 za = *reinterpret_cast<const float4 *>(st + 272 + 36 * gsel + 4 * kb);
            const float4 zb = *reinterpret_cast<const float4 *>(st + 272 + 36 * gsel + 16 + 4 * kb);
            const float v8[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
            const float z8[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
#pragma unroll
            for (int s = 0; s < HQ; s++) {
                const float4 pa = *reinterpret_cast<const float4 *>(px + (s * 4 + (r >> 2)) * PXR + 4 * kb);
                const float4 pb =
                    *reinterpret_cast<const float4 *>(px + (s * 4 + (r >> 2)) * PXR + 16 + 4 * kb);
                const float p8[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    split2(p8[2 * e2] * v8[2 * e2], p8[2 * e2 + 1] * v8[2 * e2 + 1], hi[e2], lo[e2]);
                    zt[s] = fmaf(p8[2 * e2], z8[2 * e2], fmaf(p8[2 * e2 + 1], z8[2 * e2 + 1], zt[s]));
                }
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    const uint32_t recv = dppu<0xB1>(hl ? hi[e2] : lo[e2]);  // from lane r ^ 1
                    a0[s][e2] = hl ? recv : hi[e2];
                    a1[s][e2] = hl ? lo[e2] : recv;
                }
            }
        }
        const Codes8 v0(Gr.vc[0]), v1(Gr.vc[1]), v2(Gr.vc[2]), v3(Gr.vc[3]);
        __builtin_amdgcn_s_setprio(1);
        // two tiles in flight: a product's result is read after the next
        // product has issued
#pragma unroll
        for (int n = 0; n < 8; n += 2) {
            const u4_t bv0 = {v0[n], v1[n], v2[n], v3[n]};
            const u4_t bv1 = {v0[n + 1], v1[n + 1], v2[n + 1], v3[n + 1]};
            const int i = 2 * ((n >> 1) & 1);
#pragma unroll
            for (int s = 0; s < HQ; s++) {
                const f4_t c0 = mfma_f16(n < 4 ? a0[s] : a1[s], bv0, f4_t{0, 0, 0, 0});
                const f4_t c1 = mfma_f16(n < 4 ? a0[s] : a1[s], bv1, f4_t{0, 0, 0, 0});
                acc[s][n] += c0[i] + c0[i + 1];
                acc[s][n + 1] += c1[i] + c1[i + 1];
            }
        }
        __builtin_amdgcn_s_setprio(1);
    };

    // (an empty range only occurs in a graph-replayed step: the split then
    // writes an empty partial, m = -inf and l = 0)
    if (g0 < g1) {
        GroupRegs<KHE> gb;
        for (int gi = g0;;) {
            load_group<KH>(gb, rs_of(gi + 1), O, (gi + 1) & 3);
            process(ga);
            if (++gi >= g1) break;
            load_group<KH>(ga, rs_of(gi + 1), O, (gi + 1) & 3);
            process(gb);
            if (++gi >= g1) break;
        }
    }

    // --- partials: lane (r, R) owns head head_of(R, s), channels 16 n + r ---
#pragma unroll
    for (int s = 0; s < HQ; s++) {
        const float l = row_sum(l_part[s]);
        // zt: lanes (4 R' + 2 (cg & 1) + (cg >> 1), kb) hold head row R', Value
        // group cg: sum over kb
        float z = zt[s];
        z += shfl_xor(z, 16);
        z += shfl_xor(z, 32);
        float zg[4];
#pragma unroll
        for (int cg = 0; cg < 4; cg++)
            zg[cg] = shfl(z, 4 * kb + 2 * (cg & 1) + (cg >> 1));
        const int hh = head_of<G>(kb, s);
        if (s == 0 && NW > 1) wave_sync();  // this wave's reads of its LDS region are done
        if (G >= 4 || kb < G) {
#pragma unroll
            for (int n = 0; n < 8; n++)
                put_acc(hh, 16 * n + r, acc[s][n] * ldexpf(1.0f, 24 - 2 * code_sig(n)) + zg[n >> 1]);
            if (r == 0) put_ml(hh, m_run[s] - (float)Eu, l);
        }
    }
    merge();
}

// Split combine.  A workgroup covers one output row (sequence, query head)
// or a slice of it: 32 lanes x CPL channels, so D / (32 CPL) workgroups per
// row (many rows: CPL = 4, one workgroup per row; few rows with many splits:
// CPL = 1, four).  Every load is issued first: thread (stripe, lane) reads
// its channels from splits stripe, stripe + 8, ... (at most PER of them) into
// registers, and the split statistics (m, l) two per thread; then the
// maximum, the weights exp2(m_s - M) into LDS, the weighted sums of the eight
// stripes and one LDS reduction.  Row bq merges n partials (n == 0: a
// sequence without tokens, the row is zero).
constexpr int kCombineThreads = 256;
constexpr int kCombineStripes = kCombineThreads / 32;
constexpr int kCombinePerMax = (kMaxCombine + kCombineStripes - 1) / kCombineStripes;
static_assert(2 * kCombineThreads >= kMaxCombine, "two split statistics per thread");
template <int CPL>
struct CombineVec;
template <>
struct CombineVec<1> { typedef float T; };
template <>
struct CombineVec<4> { typedef f4_t T; };
template <int PER, int CPL>
__device__ __forceinline__ void combine_body(const float *__restrict__ ws_ml,
                                             const float *__restrict__ ws_acc,
                                             float *__restrict__ out, int n, int max_splits,
                                             size_t bq, int slice) {
    typedef typename CombineVec<CPL>::T vec;
    __shared__ float wsh[kMaxCombine];
    __shared__ float red[4], dred[4];
    __shared__ vec part[kCombineStripes][32];
    const int t = threadIdx.x, wv = t >> 6, ln = t & 63;
    const int c = t & 31, stripe = t >> 5;
    vec *o = reinterpret_cast<vec *>(out + bq * D + 32 * CPL * slice) + c;
    if (n == 0) {
        if (t < 32) *o = vec{};
        return;
    }
    const float *ml = ws_ml + bq * max_splits * 2;
    const vec *a = reinterpret_cast<const vec *>(ws_acc + bq * max_splits * D + 32 * CPL * slice) + c;
    vec x[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int sp = stripe + kCombineStripes * i;
        x[i] = sp < n ? a[(size_t)sp * (D / CPL)] : vec{};
    }
    const int s1 = t + kCombineThreads;
    const float m0 = t < n ? ml[2 * t] : -INFINITY, l0 = t < n ? ml[2 * t + 1] : 0.0f;
    const float m1 = s1 < n ? ml[2 * s1] : -INFINITY, l1 = s1 < n ? ml[2 * s1 + 1] : 0.0f;
    const float m = wave_max(fmaxf(m0, m1));
    if (ln == 0) red[wv] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float w0 = t < n ? __builtin_amdgcn_exp2f(m0 - M) : 0.0f;
    const float w1 = s1 < n ? __builtin_amdgcn_exp2f(m1 - M) : 0.0f;
    if (t < n) wsh[t] = w0;
    if (s1 < n) wsh[s1] = w1;
    const float den = wave_sum(fmaf(w0, l0, w1 * l1));
    if (ln == 0) dred[wv] = den;
    __syncthreads();
    vec acc{};
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int sp = stripe + kCombineStripes * i;
        if (sp < n) acc += wsh[sp] * x[i];
    }
    part[stripe][c] = acc;
    __syncthreads();
    if (t < 32) {
        vec r = part[0][t];
#pragma unroll
        for (int i = 1; i < kCombineStripes; i++) r += part[i][t];
        *o = r / ((dred[0] + dred[1]) + (dred[2] + dred[3]));
    }
}

// Combine kernel shape for rows x splits: (PER, CPL) and workgroups per row.
struct CombineShape {
    int per, cpl;
};
inline CombineShape combine_shape(int rows, int max_n) {
    CombineShape c;
    c.cpl = rows >= 256 ? 4 : 1;
    c.per = max_n <= 8 * kCombineStripes ? 8 : kCombinePerMax;
    return c;
}

}  // namespace
}  // namespace kvq
