// kvq_quantize.hip -- page quantization, window flush and append kernels
// (gfx950) and their launchers.  The quantizer itself (channel ranking, Key
// and Value codes, packing) is in kvq_quantize_core.h.
#include "kvq_quantize_core.h"

namespace kvq {
namespace {

using namespace qz;

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
