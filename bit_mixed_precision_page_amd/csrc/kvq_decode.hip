// kvq_decode.hip -- split-K GQA decode attention over the packed cache (gfx950).
//
// Grid (split, KV head, sequence).  A page split streams its pages: the
// packed Key planes are unpacked and dequantized in registers (code =
// lo + 4 hi for boosted channels, x = code * s + z; Kitty abstract: two
// uniform 2-bit planes per mixed-precision Key page), scores for the whole
// query group of the KV head are formed from one read of the page (one Key
// head shared by several query heads, notes.yuuk.io open questions), an
// online softmax keeps (m, l) per head, and Value codes are dequantized into
// the output accumulators (MiniKV summary: unpack fused into the decode
// matmul).  The window split reads the exact window tokens.  A combine
// kernel merges the splits with a log-sum-exp rescale.
#include <cmath>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <int DT>
__device__ __forceinline__ float dec(uint16_t h) {
    if constexpr (DT == F16) {
        return (float)__builtin_bit_cast(_Float16, h);
    } else {
        return __uint_as_float((uint32_t)h << 16);
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int DT, int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint8_t *__restrict__ cache, const uint16_t *__restrict__ q, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int Hkv, int max_pages, uint32_t page_bytes, int k,
    size_t res_base, int n_pages, int n_res, int page_splits, int pps, int max_splits,
    float qscale) {
    constexpr int NH = (G + 1) / 2;  // heads per thread (two thread halves)
    __shared__ float qs[G][D];
    __shared__ float kS[P / GK][D], kZ[P / GK][D];
    __shared__ float vS[D / GV][P], vZ[D / GV][P];
    __shared__ int colj[D];
    __shared__ float sc[G][P];
    __shared__ float m_run[G], l_run[G], alpha[G];

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int unit = b * Hkv + h;
    const int Hq = Hkv * G;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = tid & 127, hs = tid >> 7;
    const PageLayout Ly = page_layout(k);

    for (int i = tid; i < G * D; i += kThreads) {
        int hh = i / D, c = i % D;
        qs[hh][c] = dec<DT>(q[((size_t)b * Hq + h * G + hh) * D + c]) * qscale;
    }
    if (tid < G) {
        m_run[tid] = -INFINITY;
        l_run[tid] = 0.0f;
    }
    float acc[NH];
#pragma unroll
    for (int j = 0; j < NH; j++) acc[j] = 0.0f;
    __syncthreads();

    // Softmax step over the scores in sc (one value per token; -inf = absent).
    auto softmax_step = [&]() {
        for (int hh = wave; hh < G; hh += 4) {
            float a = sc[hh][lane], c2 = sc[hh][lane + 64];
            float mx = wave_max(fmaxf(a, c2));
            float mold = m_run[hh];
            float mnew = fmaxf(mold, mx);
            float pa = exp2f(a - mnew), pb = exp2f(c2 - mnew);
            sc[hh][lane] = pa;
            sc[hh][lane + 64] = pb;
            float ls = wave_sum(pa + pb);
            if (lane == 0) {
                float al = exp2f(mold - mnew);
                alpha[hh] = al;
                l_run[hh] = l_run[hh] * al + ls;
                m_run[hh] = mnew;
            }
        }
    };

    if (split < page_splits) {
        const int p0 = split * pps;
        const int p1 = min(n_pages, p0 + pps);
        for (int p = p0; p < p1; p++) {
            const uint8_t *pg = cache + ((size_t)unit * max_pages + p) * page_bytes;
            const uint16_t *ksg = reinterpret_cast<const uint16_t *>(pg + Ly.ks);
            const uint16_t *kzg = reinterpret_cast<const uint16_t *>(pg + Ly.kz);
            const uint16_t *vsg = reinterpret_cast<const uint16_t *>(pg + Ly.vs);
            const uint16_t *vzg = reinterpret_cast<const uint16_t *>(pg + Ly.vz);
            for (int i = tid; i < (P / GK) * D; i += kThreads) {
                kS[i / D][i % D] = dec<DT>(ksg[i]);
                kZ[i / D][i % D] = dec<DT>(kzg[i]);
                vS[i / P][i % P] = dec<DT>(vsg[i]);
                vZ[i / P][i % P] = dec<DT>(vzg[i]);
            }
            if (tid < D) colj[tid] = -1;
            __syncthreads();
            if (tid < k) colj[pg[Ly.kidx + tid]] = tid;
            __syncthreads();

            // Scores: thread (token row, head half).
            if (hs < G) {
                const int t = row, g = t / GK;
                uint32_t lw[8], hw[8];
                const uint32_t *lp = reinterpret_cast<const uint32_t *>(pg + Ly.klo + t * 32);
#pragma unroll
                for (int i = 0; i < 8; i++) lw[i] = lp[i];
                const uint32_t *hp = reinterpret_cast<const uint32_t *>(pg + Ly.khi + t * (k / 4));
#pragma unroll
                for (int i = 0; i < 8; i++) hw[i] = i < k / 16 ? hp[i] : 0u;
                float s[NH];
#pragma unroll
                for (int j = 0; j < NH; j++) s[j] = 0.0f;
                for (int c = 0; c < D; c++) {
                    uint32_t code = (lw[c >> 4] >> (2 * (c & 15))) & 3u;
                    int j = colj[c];
                    if (j >= 0) code += 4u * ((hw[j >> 4] >> (2 * (j & 15))) & 3u);
                    float kh = fmaf((float)code, kS[g][c], kZ[g][c]);
#pragma unroll
                    for (int jj = 0; jj < NH; jj++) {
                        int hh = hs + 2 * jj;
                        if (hh < G) s[jj] = fmaf(qs[hh][c], kh, s[jj]);
                    }
                }
#pragma unroll
                for (int jj = 0; jj < NH; jj++) {
                    int hh = hs + 2 * jj;
                    if (hh < G) sc[hh][t] = s[jj];
                }
            }
            __syncthreads();
            softmax_step();
            __syncthreads();

            // P.V: thread (channel row, head half).
            if (hs < G) {
                const int c = row, n = c >> 4, cl = c & 15, cg = c / GV;
#pragma unroll
                for (int jj = 0; jj < NH; jj++) {
                    int hh = hs + 2 * jj;
                    if (hh < G) acc[jj] *= alpha[hh];
                }
                for (int s = 0; s < P / 32; s++) {
                    for (int G4 = 0; G4 < 4; G4++) {
                        uint4 blk = *reinterpret_cast<const uint4 *>(pg + Ly.vc + 1024 * s +
                                                                     16 * (16 * G4 + cl));
                        uint32_t wds[4] = {blk.x, blk.y, blk.z, blk.w};
#pragma unroll
                        for (int w = 0; w < 4; w++) {
                            int t0 = 32 * s + (w < 2 ? 4 * G4 + 2 * w : 16 + 4 * G4 + 2 * (w - 2));
                            float c0 = (float)((wds[w] >> (2 * n)) & 3u);
                            float c1 = (float)((wds[w] >> (16 + 2 * n)) & 3u);
                            float v0 = fmaf(c0, vS[cg][t0], vZ[cg][t0]);
                            float v1 = fmaf(c1, vS[cg][t0 + 1], vZ[cg][t0 + 1]);
#pragma unroll
                            for (int jj = 0; jj < NH; jj++) {
                                int hh = hs + 2 * jj;
                                if (hh < G)
                                    acc[jj] = fmaf(sc[hh][t0 + 1], v1, fmaf(sc[hh][t0], v0, acc[jj]));
                            }
                        }
                    }
                }
            }
            __syncthreads();
        }
    } else {
        // Window split: the newest n_res tokens, exact.
        const uint16_t *kw = reinterpret_cast<const uint16_t *>(cache + res_base +
                                                                (size_t)unit * 2 * R * D * 2);
        const uint16_t *vw = kw + (size_t)R * D;
        if (hs < G) {
            const int t = row;
            float s[NH];
#pragma unroll
            for (int j = 0; j < NH; j++) s[j] = t < n_res ? 0.0f : -INFINITY;
            if (t < n_res) {
                for (int c = 0; c < D; c++) {
                    float kh = dec<DT>(kw[t * D + c]);
#pragma unroll
                    for (int jj = 0; jj < NH; jj++) {
                        int hh = hs + 2 * jj;
                        if (hh < G) s[jj] = fmaf(qs[hh][c], kh, s[jj]);
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < NH; jj++) {
                int hh = hs + 2 * jj;
                if (hh < G) sc[hh][t] = s[jj];
            }
        }
        __syncthreads();
        softmax_step();
        __syncthreads();
        if (hs < G) {
            const int c = row;
            for (int t = 0; t < n_res; t++) {
                float v = dec<DT>(vw[t * D + c]);
#pragma unroll
                for (int jj = 0; jj < NH; jj++) {
                    int hh = hs + 2 * jj;
                    if (hh < G) acc[jj] = fmaf(sc[hh][t], v, acc[jj]);
                }
            }
        }
        __syncthreads();
    }

    // Partials of this split.
    if (hs < G) {
#pragma unroll
        for (int jj = 0; jj < NH; jj++) {
            int hh = hs + 2 * jj;
            if (hh < G) {
                size_t bq = (size_t)b * Hq + h * G + hh;
                ws_acc[(bq * max_splits + split) * D + row] = acc[jj];
            }
        }
    }
    if (tid < G) {
        size_t bq = (size_t)b * Hq + h * G + tid;
        ws_ml[(bq * max_splits + split) * 2 + 0] = m_run[tid];
        ws_ml[(bq * max_splits + split) * 2 + 1] = l_run[tid];
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

template <int DT>
hipError_t launch_g(const Geometry &G, const uint8_t *cache, const uint16_t *q, float *ml,
                    float *acc, const DecodePlan &pl, hipStream_t st) {
    dim3 grid(pl.total_splits, G.Hkv, G.B);
    float qscale = G.scale * kLog2e;
#define KVQ_LAUNCH(GG)                                                                         \
    hipLaunchKernelGGL((decode_split_kernel<DT, GG>), grid, dim3(kThreads), 0, st, cache, q, ml, \
                       acc, G.Hkv, G.max_pages, G.page_bytes, G.k, G.res_base, pl.n_pages,     \
                       pl.n_res, pl.page_splits, pl.pages_per_split, pl.max_splits, qscale)
    switch (G.g) {
        case 1: KVQ_LAUNCH(1); break;
        case 2: KVQ_LAUNCH(2); break;
        case 4: KVQ_LAUNCH(4); break;
        case 8: KVQ_LAUNCH(8); break;
        case 16: KVQ_LAUNCH(16); break;
        default: return hipErrorInvalidValue;
    }
#undef KVQ_LAUNCH
    return hipGetLastError();
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
    e = G.dtype == F16 ? launch_g<F16>(G, cache, q, ml, acc, pl, st)
                       : launch_g<BF16>(G, cache, q, ml, acc, pl, st);
    if (e != hipSuccess) return e;
    if (ev_after && (e = hipEventRecord(ev_after, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3(G.B * G.Hq), dim3(D), 0, st, ml, acc, out,
                       pl.total_splits, pl.max_splits);
    return hipGetLastError();
}

}  // namespace kvq
