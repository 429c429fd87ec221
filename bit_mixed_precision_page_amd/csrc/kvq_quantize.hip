// kvq_quantize.hip -- page quantization, window flush and append (gfx950).
//
// One workgroup of 256 threads quantizes one page (128 tokens x 128 channels
// of one sequence and KV head):
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
#include "kvq_internal.h"

namespace kvq {
namespace {

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

__device__ __forceinline__ uint32_t quant_code(float x, float zf, float inv, int L) {
    if (inv == 0.0f) return 0u;  // s == 0: every code is 0
    float d = __fsub_rn(x, zf);
    float t = __fmul_rn(d, inv);
    float r = rintf(t);
    r = r < 0.0f ? 0.0f : r;
    r = r > (float)L ? (float)L : r;
    return (uint32_t)r;
}

// One page: K and V rows [P][D] at ks / vs, the packed page written to pg;
// rel: [D] channel relevance (query-aware ranking) or null (magnitude).
template <int DT>
__device__ __forceinline__ void quantize_page_body(uint8_t *__restrict__ pg,
                                                   const uint16_t *__restrict__ ks,
                                                   const uint16_t *__restrict__ vs, int k,
                                                   const float *__restrict__ rel) {
    __shared__ __align__(16) uint16_t tile[P * kRowPad];
    __shared__ __align__(16) uint8_t codes[P * D];
    __shared__ uint32_t amax[2][D];  // |K| bits, or fp32 bits of two group ranges
    __shared__ uint64_t keys[D];
    __shared__ uint8_t boosted[D];
    __shared__ uint8_t idx[D];
    __shared__ uint64_t mask0;

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

    // 2. Key column statistics: thread (c, half) covers groups 2 half, 2 half + 1.
    const int c = tid & (D - 1);
    const int half = tid >> 7;
    float glo[2], ghi[2];
    uint32_t am = 0;
#pragma unroll
    for (int gg = 0; gg < 2; gg++) {
        int g = 2 * half + gg;
        uint16_t h0 = tile[(g * GK) * kRowPad + c];
        float lo = dec<DT>(h0), hi = lo;
        am = max(am, (uint32_t)(h0 & 0x7fffu));
        for (int t = 1; t < GK; t++) {
            uint16_t h = tile[(g * GK + t) * kRowPad + c];
            float x = dec<DT>(h);
            lo = x < lo ? x : lo;
            hi = x > hi ? x : hi;
            am = max(am, (uint32_t)(h & 0x7fffu));
        }
        glo[gg] = lo;
        ghi[gg] = hi;
    }
    if (rel) {
        // ranges of this thread's groups 2 half and 2 half + 1, summed pairwise
        amax[half][c] = __float_as_uint(
            __fadd_rn(__fsub_rn(ghi[0], glo[0]), __fsub_rn(ghi[1], glo[1])));
    } else {
        amax[half][c] = am;
    }
    __syncthreads();
    if (tid < D) {
        uint64_t sc;
        if (rel) {
            const float diff = __fadd_rn(__uint_as_float(amax[0][tid]), __uint_as_float(amax[1][tid]));
            sc = __float_as_uint(__fmul_rn(diff, rel[tid])) & 0x7fffffffu;
        } else {
            sc = max(amax[0][tid], amax[1][tid]);
        }
        keys[tid] = (sc << 8) | (uint64_t)(255 - tid);
    }
    __syncthreads();

    // 3. Top-k by rank count; ascending list through wave ballots.
    if (tid < D) {
        const uint64_t my = keys[tid];
        int rank = 0;
        for (int j = 0; j < D; j++) rank += keys[j] > my ? 1 : 0;
        bool b = rank < k;
        boosted[tid] = b ? 1 : 0;
        uint64_t m = __ballot(b);  // waves 0 and 1 are fully active here
        if (tid == 0) mask0 = m;
    }
    __syncthreads();
    if (tid < D) {
        uint64_t m = __ballot(boosted[tid] != 0);
        int lane = tid & 63;
        int pos = __popcll(m & ((1ull << lane) - 1ull)) + (tid >= 64 ? __popcll(mask0) : 0);
        if (boosted[tid]) idx[pos] = (uint8_t)tid;
    }
    __syncthreads();

    // 4. Key codes and metadata.
#pragma unroll
    for (int gg = 0; gg < 2; gg++) {
        int g = 2 * half + gg;
        int L = boosted[c] ? 15 : 3;
        uint16_t sb, zb;
        float zf, inv;
        group_params<DT>(glo[gg], ghi[gg], L, sb, zb, zf, inv);
        reinterpret_cast<uint16_t *>(pg + Ly.ks)[g * D + c] = sb;
        reinterpret_cast<uint16_t *>(pg + Ly.kz)[g * D + c] = zb;
        for (int t = 0; t < GK; t++) {
            float x = dec<DT>(tile[(g * GK + t) * kRowPad + c]);
            codes[(g * GK + t) * D + c] = (uint8_t)quant_code(x, zf, inv, L);
        }
    }
    if (tid < k / 16)
        reinterpret_cast<uint4 *>(pg + Ly.kidx)[tid] = reinterpret_cast<const uint4 *>(idx)[tid];
    __syncthreads();

    // 5. Pack the lo plane (16 B per thread) and the hi plane (k/4 B per token).
    {
        int t = tid >> 1, c0 = (tid & 1) * 64;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint32_t acc = 0;
            const uint8_t *src = &codes[t * D + c0 + 16 * q];
#pragma unroll
            for (int e = 0; e < 16; e++) acc |= ((uint32_t)src[e] & 3u) << (2 * e);
            w[q] = acc;
        }
        *reinterpret_cast<uint4 *>(pg + Ly.klo + t * 32 + (tid & 1) * 16) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (tid < P && k > 0) {
        int t = tid;
        uint32_t *dst = reinterpret_cast<uint32_t *>(pg + Ly.khi + t * (k / 4));
        for (int q = 0; q < k / 16; q++) {
            uint32_t acc = 0;
            for (int e = 0; e < 16; e++)
                acc |= ((uint32_t)codes[t * D + idx[16 * q + e]] >> 2) << (2 * e);
            dst[q] = acc;
        }
    }
    __syncthreads();

    // 6. Values: tile <- V, then per (token, 32-channel group) statistics.
#pragma unroll
    for (int j = 0; j < 8; j++) {
        int i = tid + kThreads * j;
        *reinterpret_cast<u4_t *>(&tile[(i >> 4) * kRowPad + (i & 15) * 8]) = vr[j];
    }
    __syncthreads();
    {
        int t = tid >> 1;
#pragma unroll
        for (int gg = 0; gg < 2; gg++) {
            int h = 2 * (tid & 1) + gg;
            const uint16_t *row = &tile[t * kRowPad + h * GV];
            float lo = dec<DT>(row[0]), hi = lo;
            for (int e = 1; e < GV; e++) {
                float x = dec<DT>(row[e]);
                lo = x < lo ? x : lo;
                hi = x > hi ? x : hi;
            }
            uint16_t sb, zb;
            float zf, inv;
            group_params<DT>(lo, hi, 3, sb, zb, zf, inv);
            reinterpret_cast<uint16_t *>(pg + Ly.vs)[h * P + t] = sb;
            reinterpret_cast<uint16_t *>(pg + Ly.vz)[h * P + t] = zb;
            for (int e = 0; e < GV; e++)
                codes[t * D + h * GV + e] = (uint8_t)quant_code(dec<DT>(row[e]), zf, inv, 3);
        }
    }
    __syncthreads();

    // 7. Pack Value codes: thread = one 16-byte block (step s, lane 16 G + cl).
    {
        int s = tid >> 6, lane = tid & 63, G = lane >> 4, cl = lane & 15;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            int t0 = 32 * s + (q < 2 ? 4 * G + 2 * q : 16 + 4 * G + 2 * (q - 2));
            uint32_t acc = 0;
#pragma unroll
            for (int n = 0; n < 8; n++) {
                acc |= (uint32_t)codes[t0 * D + 16 * n + cl] << (2 * n);
                acc |= (uint32_t)codes[(t0 + 1) * D + 16 * n + cl] << (16 + 2 * n);
            }
            w[q] = acc;
        }
        *reinterpret_cast<uint4 *>(pg + Ly.vc + 1024 * s + 16 * lane) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Dense cache: page first_page + blockIdx.x of unit blockIdx.y.
template <int DT>
__global__ __launch_bounds__(kThreads) void quantize_pages_kernel(
    uint8_t *__restrict__ cache, const uint16_t *__restrict__ k_src,
    const uint16_t *__restrict__ v_src, size_t src_unit_stride, int first_page, int n_new,
    int max_pages, uint32_t page_bytes, int k, const float *__restrict__ rel) {
    const int p = blockIdx.x;
    const int unit = blockIdx.y;
    uint8_t *pg = cache + ((size_t)unit * max_pages + first_page + p) * page_bytes;
    const uint16_t *ks = k_src + (size_t)unit * src_unit_stride + (size_t)p * P * D;
    const uint16_t *vs = v_src + (size_t)unit * src_unit_stride + (size_t)p * P * D;
    quantize_page_body<DT>(pg, ks, vs, k, rel ? rel + (size_t)unit * D : nullptr);
}

// Block pool: entry blockIdx.x of the list, KV head blockIdx.y.  The page
// goes to pool block pp.block[e] (the block holds the Hkv pages of one
// 128-token span); its source rows start at element
// pp.src[e] * src_e_stride + h * src_h_stride; the KV-head-0 workgroup
// records the block in the block table (entry tslot = seq * max_pages + page,
// which also names the relevance row of the sequence).
template <int DT>
__global__ __launch_bounds__(kThreads) void pool_pages_kernel(
    uint8_t *__restrict__ pool, int32_t *__restrict__ table, const uint16_t *__restrict__ k_src,
    const uint16_t *__restrict__ v_src, size_t src_h_stride, size_t src_e_stride, int Hkv,
    int max_pages, uint32_t page_bytes, int k, const float *__restrict__ rel,
    const PoolPages pp) {
    const int e = blockIdx.x, h = blockIdx.y;
    const int blk = pp.block[e];
    if (h == 0 && threadIdx.x == 0) table[pp.tslot[e]] = blk;
    uint8_t *pg = pool + ((size_t)blk * Hkv + h) * page_bytes;
    const size_t so = (size_t)pp.src[e] * src_e_stride + (size_t)h * src_h_stride;
    const int seq = pp.tslot[e] / max_pages;
    quantize_page_body<DT>(pg, k_src + so, v_src + so, k,
                           rel ? rel + ((size_t)seq * Hkv + h) * D : nullptr);
}

// rel[b][h][c] = sum over the g query heads h g + j (j ascending) of
// |q[b][h g + j][c]| in fp32: the relevance of one query to each Key channel.
template <int DT>
__global__ __launch_bounds__(kThreads) void query_relevance_kernel(
    const uint16_t *__restrict__ q, float *__restrict__ rel, int B, int Hq, int Hkv) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= B * Hkv * D) return;
    const int c = i % D, bh = i / D, b = bh / Hkv, h = bh % Hkv, g = Hq / Hkv;
    float acc = 0.0f;
    for (int j = 0; j < g; j++)
        acc = __fadd_rn(acc, fabsf(dec<DT>(q[((size_t)b * Hq + h * g + j) * D + c])));
    rel[i] = acc;
}

// Block pool: copy one token per (sequence, KV head) into window slot
// ps.slot[sequence] (kPoolNoSlot: the sequence takes no token).
template <int DT>
__global__ __launch_bounds__(kThreads) void pool_append_kernel(
    uint8_t *__restrict__ mem, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    int Hkv, int n_seq, size_t res_base, const PoolSlots ps) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    const int per = n_seq * Hkv * 16;
    if (i >= 2 * per) return;
    const bool isv = i >= per;
    const int j = isv ? i - per : i;
    const int unit = j >> 4, chunk = j & 15;
    const int slot = ps.slot[unit / Hkv];
    if (slot == kPoolNoSlot) return;
    const uint16_t *src = (isv ? v : k) + (size_t)unit * D + chunk * 8;
    const size_t dst = res_base + (size_t)unit * 2 * R * D * 2 + (isv ? (size_t)R * D * 2 : 0) +
                       ((size_t)slot * D + chunk * 8) * 2;
    *reinterpret_cast<uint4 *>(mem + dst) = *reinterpret_cast<const uint4 *>(src);
}

// Block pool: tokens [first, first + tail) of one sequence's K and V
// ([Hkv][n_tokens][D]) into window slots [0, tail) of that sequence.
__global__ __launch_bounds__(kThreads) void pool_window_fill_kernel(
    uint8_t *__restrict__ mem, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    int seq, int Hkv, int n_tokens, int first, int tail, size_t res_base) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    const int per = Hkv * tail * 16;
    if (i >= 2 * per) return;
    const bool isv = i >= per;
    const int j = isv ? i - per : i;
    const int h = j / (tail * 16), rem = j % (tail * 16);
    const int t = rem >> 4, chunk = rem & 15;
    const uint16_t *src = (isv ? v : k) + ((size_t)h * n_tokens + first + t) * D + chunk * 8;
    const size_t dst = res_base + (size_t)(seq * Hkv + h) * 2 * R * D * 2 +
                       (isv ? (size_t)R * D * 2 : 0) + ((size_t)t * D + chunk * 8) * 2;
    *reinterpret_cast<uint4 *>(mem + dst) = *reinterpret_cast<const uint4 *>(src);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void append_kernel(uint8_t *__restrict__ cache,
                                                          const uint16_t *__restrict__ k,
                                                          const uint16_t *__restrict__ v,
                                                          int units, size_t res_base, int slot) {
    // 16 chunks of 16 B per vector; K chunks first, then V chunks.
    int i = blockIdx.x * kThreads + threadIdx.x;
    int per = units * 16;
    if (i >= 2 * per) return;
    bool isv = i >= per;
    int j = isv ? i - per : i;
    int unit = j >> 4, chunk = j & 15;
    const uint16_t *src = (isv ? v : k) + (size_t)unit * D + chunk * 8;
    size_t dst = res_base + (size_t)unit * 2 * R * D * 2 + (isv ? (size_t)R * D * 2 : 0) +
                 ((size_t)slot * D + chunk * 8) * 2;
    *reinterpret_cast<uint4 *>(cache + dst) = *reinterpret_cast<const uint4 *>(src);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void quantize_groups_kernel(
    const uint16_t *__restrict__ x, int n_groups, int group_len, int L, uint16_t *s,
    uint16_t *z, uint8_t *codes) {
    int gidx = blockIdx.x * kThreads + threadIdx.x;
    if (gidx >= n_groups) return;
    const uint16_t *xs = x + (size_t)gidx * group_len;
    float lo = dec<DT>(xs[0]), hi = lo;
    for (int i = 1; i < group_len; i++) {
        float v = dec<DT>(xs[i]);
        lo = v < lo ? v : lo;
        hi = v > hi ? v : hi;
    }
    uint16_t sb, zb;
    float zf, inv;
    group_params<DT>(lo, hi, L, sb, zb, zf, inv);
    s[gidx] = sb;
    z[gidx] = zb;
    for (int i = 0; i < group_len; i++)
        codes[(size_t)gidx * group_len + i] = (uint8_t)quant_code(dec<DT>(xs[i]), zf, inv, L);
}

}  // namespace

hipError_t launch_quantize_pages(const Geometry &G, uint8_t *cache, const uint16_t *k_src,
                                 const uint16_t *v_src, size_t src_unit_stride,
                                 int first_page, int n_new, const float *rel,
                                 hipStream_t stream) {
    if (n_new <= 0) return hipSuccess;
    dim3 grid(n_new, G.B * G.Hkv);
    if (G.dtype == F16)
        hipLaunchKernelGGL(quantize_pages_kernel<F16>, grid, dim3(kThreads), 0, stream, cache,
                           k_src, v_src, src_unit_stride, first_page, n_new, G.max_pages,
                           G.page_bytes, G.k, rel);
    else
        hipLaunchKernelGGL(quantize_pages_kernel<BF16>, grid, dim3(kThreads), 0, stream, cache,
                           k_src, v_src, src_unit_stride, first_page, n_new, G.max_pages,
                           G.page_bytes, G.k, rel);
    return hipGetLastError();
}

hipError_t launch_flush_window(const Geometry &G, uint8_t *cache, int page, const float *rel,
                               hipStream_t stream) {
    const uint16_t *kw = reinterpret_cast<const uint16_t *>(cache + G.res_base);
    const uint16_t *vw = kw + (size_t)R * D;
    return launch_quantize_pages(G, cache, kw, vw, (size_t)2 * R * D, page, 1, rel, stream);
}

hipError_t launch_query_relevance(int dtype, const uint16_t *q, float *rel, int B, int Hq,
                                  int Hkv, hipStream_t stream) {
    const int n = B * Hkv * D;
    dim3 grid((n + kThreads - 1) / kThreads);
    if (dtype == F16)
        hipLaunchKernelGGL(query_relevance_kernel<F16>, grid, dim3(kThreads), 0, stream, q, rel,
                           B, Hq, Hkv);
    else
        hipLaunchKernelGGL(query_relevance_kernel<BF16>, grid, dim3(kThreads), 0, stream, q, rel,
                           B, Hq, Hkv);
    return hipGetLastError();
}

hipError_t launch_append(const Geometry &G, uint8_t *cache, const uint16_t *k,
                         const uint16_t *v, int slot, hipStream_t stream) {
    int units = G.B * G.Hkv;
    int n = 2 * units * 16;
    dim3 grid((n + kThreads - 1) / kThreads);
    if (G.dtype == F16)
        hipLaunchKernelGGL(append_kernel<F16>, grid, dim3(kThreads), 0, stream, cache, k, v,
                           units, G.res_base, slot);
    else
        hipLaunchKernelGGL(append_kernel<BF16>, grid, dim3(kThreads), 0, stream, cache, k, v,
                           units, G.res_base, slot);
    return hipGetLastError();
}

hipError_t launch_pool_pages(const Geometry &G, uint8_t *pool, int32_t *table,
                             const uint16_t *k_src, const uint16_t *v_src, size_t src_h_stride,
                             size_t src_e_stride, const PoolPages &pp, const float *rel,
                             hipStream_t stream) {
    if (pp.n <= 0) return hipSuccess;
    dim3 grid(pp.n, G.Hkv);
    if (G.dtype == F16)
        hipLaunchKernelGGL(pool_pages_kernel<F16>, grid, dim3(kThreads), 0, stream, pool, table,
                           k_src, v_src, src_h_stride, src_e_stride, G.Hkv, G.max_pages,
                           G.page_bytes, G.k, rel, pp);
    else
        hipLaunchKernelGGL(pool_pages_kernel<BF16>, grid, dim3(kThreads), 0, stream, pool, table,
                           k_src, v_src, src_h_stride, src_e_stride, G.Hkv, G.max_pages,
                           G.page_bytes, G.k, rel, pp);
    return hipGetLastError();
}

hipError_t launch_pool_append(const Geometry &G, uint8_t *mem, const uint16_t *k,
                              const uint16_t *v, const PoolSlots &ps, hipStream_t stream) {
    const int n = 2 * G.B * G.Hkv * 16;
    dim3 grid((n + kThreads - 1) / kThreads);
    if (G.dtype == F16)
        hipLaunchKernelGGL(pool_append_kernel<F16>, grid, dim3(kThreads), 0, stream, mem, k, v,
                           G.Hkv, G.B, G.res_base, ps);
    else
        hipLaunchKernelGGL(pool_append_kernel<BF16>, grid, dim3(kThreads), 0, stream, mem, k, v,
                           G.Hkv, G.B, G.res_base, ps);
    return hipGetLastError();
}

hipError_t launch_pool_window_fill(const Geometry &G, uint8_t *mem, const uint16_t *k,
                                   const uint16_t *v, int seq, int n_tokens, int first, int tail,
                                   hipStream_t stream) {
    if (tail <= 0) return hipSuccess;
    const int n = 2 * G.Hkv * tail * 16;
    hipLaunchKernelGGL(pool_window_fill_kernel, dim3((n + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, stream, mem, k, v, seq, G.Hkv, n_tokens, first, tail,
                       G.res_base);
    return hipGetLastError();
}

hipError_t launch_quantize_groups(int dtype, int L, const uint16_t *x, int n_groups,
                                  int group_len, uint16_t *s, uint16_t *z, uint8_t *codes,
                                  hipStream_t stream) {
    if (n_groups <= 0) return hipSuccess;
    dim3 grid((n_groups + kThreads - 1) / kThreads);
    if (dtype == F16)
        hipLaunchKernelGGL(quantize_groups_kernel<F16>, grid, dim3(kThreads), 0, stream, x,
                           n_groups, group_len, L, s, z, codes);
    else
        hipLaunchKernelGGL(quantize_groups_kernel<BF16>, grid, dim3(kThreads), 0, stream, x,
                           n_groups, group_len, L, s, z, codes);
    return hipGetLastError();
}

}  // namespace kvq
