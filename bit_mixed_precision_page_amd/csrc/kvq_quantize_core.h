// kvq_quantize_core.h -- device code of the page quantizer (gfx950): one
// workgroup of kThreads threads turns 128 tokens x 128 channels of one
// sequence and KV head into a packed page.  Used by the quantize, flush and
// pool kernels and by the merge launch of a graph-replayed decode step, which
// flushes a window that its step has just filled.
//
//   * Key channel ranking (Kitty abstract: rank Key channels, keep a small
//     fraction at higher precision; notes.yuuk.io "KV cache quantization",
//     open questions: the heuristic is magnitude based): score = max |K| over
//     the page as sign-cleared bits, ties to the lower channel, top k by an
//     exact rank count.  With a relevance vector (MixKVQ abstract: the
//     channel's quantization difficulty and its relevance to the query) the
//     score is |(sum of the channel's four Key-group ranges) * relevance|;
//   * Keys per channel over 32-token groups, Values per token over
//     32-channel groups, asymmetric min/max (KIVI explainer, section 3);
//     boosted channels with 4 bits split into a lo and a hi 2-bit plane;
//   * packing into the page layout with 16-byte stores.
// Code decisions use IEEE fp32 with correctly rounded division (never rcp)
// and round-half-even, one operation at a time.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace qz {
constexpr int kThreads = 256;
// 16 bytes as a native vector, so that arrays of them stay in registers
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
constexpr int kRowPad = 136;  // LDS row stride in u16 (272 B) to spread banks

template <int DT>
__device__ __forceinline__ float dec(uint16_t h) {
    if constexpr (DT == F16) {
        return (float)__builtin_bit_cast(_Float16, h);
    } else {
        return __uint_as_float((uint32_t)h << 16);
    }
}

template <int DT>
__device__ __forceinline__ uint16_t enc_rne(float f) {
    if constexpr (DT == F16) {
        return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, RNE
    } else {
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
        u += 0x7fffu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
}

// Quantizer Q(x; L) on a group already reduced to (lo, hi): returns the
// stored scale and zero and the fp32 values the code decision uses.
template <int DT>
__device__ __forceinline__ void group_params(float lo, float hi, int L, uint16_t &s_bits,
                                             uint16_t &z_bits, float &zf, float &inv) {
    if (lo == 0.0f) lo = 0.0f;  // a zero minimum is stored as +0
    float range = hi - lo;
    float s32 = __fdiv_rn(range, (float)L);
    s_bits = enc_rne<DT>(s32);
    z_bits = enc_rne<DT>(lo);  // exact: lo is a stored value
    float sf = dec<DT>(s_bits);
    zf = dec<DT>(z_bits);
    inv = sf == 0.0f ? 0.0f : __fdiv_rn(1.0f, sf);
}

// code = clamp(rint((x - z) * inv), 0, L).  No branch for s == 0: then
// inv == 0 and x - z is finite and >= 0 (z is the group minimum, the range is
// finite), so the product is +-0 and the code 0, as the definition gives.
__device__ __forceinline__ uint32_t quant_code(float x, float zf, float inv, int L) {
    float d = __fsub_rn(x, zf);
    float t = __fmul_rn(d, inv);
    float r = __builtin_amdgcn_fmed3f(rintf(t), 0.0f, (float)L);
    return (uint32_t)r;
}

// Decode the two stored values packed in one 32-bit word (lower address first).
template <int DT>
__device__ __forceinline__ float dec_lo(uint32_t w) { return dec<DT>((uint16_t)(w & 0xffffu)); }
template <int DT>
__device__ __forceinline__ float dec_hi(uint32_t w) { return dec<DT>((uint16_t)(w >> 16)); }

// Running min / max.  The maximum keeps the first of equal values, so a zero
// maximum keeps the sign it had first (as the element-by-element definition
// does: the sign reaches the stored scale through max - min).  The minimum's
// zero sign never matters (a zero minimum is stored as +0, and the query-aware
// score takes |.| of its ranges), so it uses the plain min instruction.
__device__ __forceinline__ void minmax(float x, float &lo, float &hi) {
    lo = __builtin_fminf(x, lo);
    hi = x > hi ? x : hi;
}

// One page: K and V rows [P][D] at ks / vs, the packed page written to pg;
// rel: [D] channel relevance (query-aware ranking) or null (magnitude).
//
// Work split of the 256 threads (4 waves):
//   Key statistics and codes by columns: wave g owns Key group g (32
//     tokens), lane p the channel pair (2p, 2p + 1); its 64 values stay in
//     registers from the statistics to the codes.
//   Channel ranking: every thread counts the larger keys in one half.
//   K lo plane: code pairs become nibbles, lane pairs bytes, staged in LDS in
//     the page's own layout and copied out with 16-byte stores.
//   K hi plane: thread (token, half) recomputes the 4-bit codes of its half of
//     the boosted list and packs their upper bits.
//   Value statistics and codes by rows: thread (token, half) owns 64 channels
//     (two Value groups); codes are staged per (channel mod 16, token) and
//     read back in the page's V_codes order.
template <int DT>
__device__ __forceinline__ void quantize_page_body(uint8_t *__restrict__ pg,
                                                   const uint16_t *__restrict__ ks,
                                                   const uint16_t *__restrict__ vs, int k,
                                                   const float *__restrict__ rel) {
    constexpr int kRow32 = kRowPad / 2;    // tile row stride in 32-bit words
    constexpr int kVpkRow = 2 * P + 8;     // bytes per staged V row (padded: spreads banks)
    __shared__ __align__(16) uint16_t tile[P * kRowPad];  // K tile, later the V tile
    __shared__ __align__(16) float kst[2][P / GK][D];     // Key group min / max per channel
    __shared__ __align__(16) uint8_t stage[16 * kVpkRow]; // K lo plane, later V code bytes
    __shared__ __align__(16) float2 hpar[P / GK][D];      // (zf, inv) of boosted channels, by list slot
    __shared__ __align__(16) uint64_t keys[D];
    __shared__ __align__(16) int rankp[2][D];
    __shared__ uint8_t boosted[D];
    __shared__ __align__(16) uint8_t idx[D];
    __shared__ int8_t jpos[D];
    __shared__ int nbelow;

    const int tid = threadIdx.x;
    const PageLayout Ly = page_layout(k);

    // 1. Issue every load of the K and V tiles (16 B per thread per step).
    u4_t kr[8], vr[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        int i = tid + kThreads * j;  // 16-byte chunk: row i / 16, 8 channels (i % 16)
        kr[j] = reinterpret_cast<const u4_t *>(ks)[i];
        vr[j] = reinterpret_cast<const u4_t *>(vs)[i];
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
        int i = tid + kThreads * j;
        *reinterpret_cast<u4_t *>(&tile[(i >> 4) * kRowPad + (i & 15) * 8]) = kr[j];
    }
    __syncthreads();

    // 2. Key statistics: wave g = Key group g, lane p = channels 2p, 2p + 1.
    const int p = tid & 63, g = tid >> 6;
    uint32_t kw[GK];
    const uint32_t *tile32 = reinterpret_cast<const uint32_t *>(tile);
#pragma unroll
    for (int t = 0; t < GK; t++) kw[t] = tile32[(g * GK + t) * kRow32 + p];
    float lo0 = dec_lo<DT>(kw[0]), hi0 = lo0, lo1 = dec_hi<DT>(kw[0]), hi1 = lo1;
#pragma unroll
    for (int t = 1; t < GK; t++) {
        minmax(dec_lo<DT>(kw[t]), lo0, hi0);
        minmax(dec_hi<DT>(kw[t]), lo1, hi1);
    }
    *reinterpret_cast<float2 *>(&kst[0][g][2 * p]) = make_float2(lo0, lo1);
    *reinterpret_cast<float2 *>(&kst[1][g][2 * p]) = make_float2(hi0, hi1);
    __syncthreads();

    // 3. Ranking keys: magnitude (largest |K| over the page, as fp32 bits of
    // the group extremes) or |(summed group ranges) * relevance|; ties go to
    // the lower channel.
    if (tid < D) {
        const int c = tid;
        uint64_t sc;
        if (rel) {
            float r[P / GK];
#pragma unroll
            for (int gg = 0; gg < P / GK; gg++) r[gg] = __fsub_rn(kst[1][gg][c], kst[0][gg][c]);
            const float diff = __fadd_rn(__fadd_rn(r[0], r[1]), __fadd_rn(r[2], r[3]));
            sc = __float_as_uint(__fmul_rn(diff, rel[c])) & 0x7fffffffu;
        } else {
            uint32_t am = 0;
#pragma unroll
            for (int gg = 0; gg < P / GK; gg++)
                am = max(am, max(__float_as_uint(kst[0][gg][c]) & 0x7fffffffu,
                                 __float_as_uint(kst[1][gg][c]) & 0x7fffffffu));
            sc = am;
        }
        keys[c] = (sc << 8) | (uint64_t)(255 - c);
    }
    __syncthreads();

    // 4. Top-k by rank count (each thread counts one half of the keys), then
    // the ascending list through wave ballots.
    {
        const int c = tid & (D - 1), part = tid >> 7;
        const uint64_t my = keys[c];
        int cnt = 0;
        const u4_t *kv = reinterpret_cast<const u4_t *>(keys + 64 * part);
#pragma unroll 8
        for (int j = 0; j < 32; j++) {
            const u4_t two = kv[j];
            const uint64_t a = (uint64_t)two[0] | ((uint64_t)two[1] << 32);
            const uint64_t b = (uint64_t)two[2] | ((uint64_t)two[3] << 32);
            cnt += (a > my ? 1 : 0) + (b > my ? 1 : 0);
        }
        rankp[part][c] = cnt;
    }
    __syncthreads();
    if (tid < D) {  // waves 0 and 1, fully active
        const bool b = rankp[0][tid] + rankp[1][tid] < k;
        boosted[tid] = b ? 1 : 0;
        const uint64_t m = __ballot(b);
        if (tid == 0) nbelow = __popcll(m);  // boosted channels below 64
        const int pos = __popcll(m & ((1ull << (tid & 63)) - 1ull));
        jpos[tid] = b ? (int8_t)pos : (int8_t)-1;  // wave 1 adds nbelow below
    }
    __syncthreads();
    if (tid < D) {
        const int pos = jpos[tid] + (tid >= 64 ? nbelow : 0);
        if (jpos[tid] >= 0) {
            idx[pos] = (uint8_t)tid;
            jpos[tid] = (int8_t)pos;
        }
    }
    __syncthreads();

    // 5. Key metadata and codes (wave g, channels 2p, 2p + 1).
    {
        const int c0 = 2 * p;
        const bool b0 = boosted[c0] != 0, b1 = boosted[c0 + 1] != 0;
        const int L0 = b0 ? 15 : 3, L1 = b1 ? 15 : 3;
        uint16_t sb0, zb0, sb1, zb1;
        float zf0, inv0, zf1, inv1;
        group_params<DT>(lo0, hi0, L0, sb0, zb0, zf0, inv0);
        group_params<DT>(lo1, hi1, L1, sb1, zb1, zf1, inv1);
        reinterpret_cast<uint32_t *>(pg + Ly.ks)[(g * D + c0) >> 1] = (uint32_t)sb0 | ((uint32_t)sb1 << 16);
        reinterpret_cast<uint32_t *>(pg + Ly.kz)[(g * D + c0) >> 1] = (uint32_t)zb0 | ((uint32_t)zb1 << 16);
        if (b0) hpar[g][jpos[c0]] = make_float2(zf0, inv0);
        if (b1) hpar[g][jpos[c0 + 1]] = make_float2(zf1, inv1);
        // lo plane: nibble (channels 2p, 2p + 1) per token, lane pairs make a
        // byte (channels 4 (p / 2) .. + 3), staged as rows of 32 bytes
#pragma unroll
        for (int t = 0; t < GK; t++) {
            const uint32_t q0 = quant_code(dec_lo<DT>(kw[t]), zf0, inv0, L0);
            const uint32_t q1 = quant_code(dec_hi<DT>(kw[t]), zf1, inv1, L1);
            const uint32_t nib = (q0 & 3u) | ((q1 & 3u) << 2);
            const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)nib, 0xB1, 0xF, 0xF, false);
            const uint32_t byte = (p & 1) ? (other | (nib << 4)) : (nib | (other << 4));
            stage[(g * GK + t) * 32 + (p >> 1)] = (uint8_t)byte;
        }
    }
    if (tid < k / 16)
        reinterpret_cast<uint4 *>(pg + Ly.kidx)[tid] = reinterpret_cast<const uint4 *>(idx)[tid];
    __syncthreads();
    *reinterpret_cast<u4_t *>(pg + Ly.klo + 16 * tid) = reinterpret_cast<const u4_t *>(stage)[tid];

    // 6. K hi plane: thread (token t, half) covers list slots
    // [half k / 2, half k / 2 + k / 2), eight per 16-bit word.
    if (k > 0) {
        const int t = tid >> 1, half = tid & 1, kg = t / GK;
        uint16_t *dst = reinterpret_cast<uint16_t *>(pg + Ly.khi + t * (k / 4) + half * (k / 8));
        for (int q = 0; q < k / 16; q++) {
            uint32_t acc = 0;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int j = half * (k / 2) + 8 * q + e;
                const float2 pr = hpar[kg][j];
                const float x = dec<DT>(tile[t * kRowPad + idx[j]]);
                acc |= (quant_code(x, pr.x, pr.y, 15) >> 2) << (2 * e);
            }
            dst[q] = (uint16_t)acc;
        }
    }
    __syncthreads();

    // 7. Values: tile <- V; thread (token t, half) reads its 64 channels.
#pragma unroll
    for (int j = 0; j < 8; j++) {
        int i = tid + kThreads * j;
        *reinterpret_cast<u4_t *>(&tile[(i >> 4) * kRowPad + (i & 15) * 8]) = vr[j];
    }
    __syncthreads();
    {
        const int t = tid >> 1, h2 = tid & 1;
        uint32_t vw[32];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const u4_t x = *reinterpret_cast<const u4_t *>(&tile[t * kRowPad + 64 * h2 + 8 * i]);
            vw[4 * i] = x[0];
            vw[4 * i + 1] = x[1];
            vw[4 * i + 2] = x[2];
            vw[4 * i + 3] = x[3];
        }
        uint32_t code[64];
#pragma unroll
        for (int gg = 0; gg < 2; gg++) {
            const uint32_t *w = vw + 16 * gg;  // channels 64 h2 + 32 gg + [0, 32)
            float lo = dec_lo<DT>(w[0]), hi = lo;
            minmax(dec_hi<DT>(w[0]), lo, hi);
#pragma unroll
            for (int e = 1; e < 16; e++) {
                minmax(dec_lo<DT>(w[e]), lo, hi);
                minmax(dec_hi<DT>(w[e]), lo, hi);
            }
            uint16_t sb, zb;
            float zf, inv;
            group_params<DT>(lo, hi, 3, sb, zb, zf, inv);
            const int hh = 2 * h2 + gg;
            reinterpret_cast<uint16_t *>(pg + Ly.vs)[hh * P + t] = sb;
            reinterpret_cast<uint16_t *>(pg + Ly.vz)[hh * P + t] = zb;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                code[32 * gg + 2 * e] = quant_code(dec_lo<DT>(w[e]), zf, inv, 3);
                code[32 * gg + 2 * e + 1] = quant_code(dec_hi<DT>(w[e]), zf, inv, 3);
            }
        }
        // byte (channel class cl = c % 16, token t, half h2): the codes of
        // channels 64 h2 + 16 m + cl, m = 0..3, at bits 2 m
#pragma unroll
        for (int cl = 0; cl < 16; cl++)
            stage[cl * kVpkRow + 2 * t + h2] =
                (uint8_t)(code[cl] | (code[16 + cl] << 2) | (code[32 + cl] << 4) | (code[48 + cl] << 6));
    }
    __syncthreads();

    // 8. V_codes: thread = one 16-byte block (32-token step s, lane 16 G + cl):
    // words hold tokens (4G, 4G + 1), (4G + 2, 4G + 3), (16 + 4G, ..), (.., 16 + 4G + 3).
    {
        const int s = tid >> 6, lane = tid & 63, G = lane >> 4, cl = lane & 15;
        const uint8_t *row = stage + cl * kVpkRow + 2 * (32 * s + 4 * G);
        const uint2 a = *reinterpret_cast<const uint2 *>(row);
        const uint2 b = *reinterpret_cast<const uint2 *>(row + 32);
        *reinterpret_cast<uint4 *>(pg + Ly.vc + 1024 * s + 16 * lane) = make_uint4(a.x, a.y, b.x, b.y);
    }
}

}  // namespace qz
}  // namespace kvq
