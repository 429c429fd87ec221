// kvq_pool.hip -- split-K GQA decode attention over a block pool: sequences
// of different lengths in one launch, pages reached through a block table.
// The per-launch plan (split counts and lengths per sequence) is a kernel
// argument; the work of a split is the same code as for the dense cache
// (kvq_decode_core.h).
#include <algorithm>

#include "kvq_decode_core.h"

namespace kvq {
namespace {

// Waves per SIMD of the pool kernel: as the dense kernel's, except eight
// heads with up to 32 boosted channels, where the block-table addressing
// would push values the group loop reads into scratch at four waves.
constexpr int pool_waves_target(int G, int KH) { return G == 8 && KH <= 1 ? 3 : waves_target(G, KH); }

// 1-D grid: the page splits of every sequence (sequence-major, then KV head,
// then split), then the window splits in the same order.
template <int DT, int G, int KH>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(pool_waves_target(G, KH)))) void pool_split_kernel(
    const uint8_t *__restrict__ mem, uint8_t *__restrict__ window_w,
    const uint16_t *__restrict__ knew, const uint16_t *__restrict__ vnew,
    const uint16_t *__restrict__ q, float *__restrict__ ws_ml, float *__restrict__ ws_acc,
    const int32_t *__restrict__ table, int Hkv, int max_pages, uint32_t page_bytes, int k,
    size_t res_base, float qscale, const PoolPlan pl) {
    int b, h, split, S;
    pool_split_of(pl, Hkv, blockIdx.x, &b, &h, &split, &S);
    b = __builtin_amdgcn_readfirstlane(b);
    const int slot = pl.slot[b] == kPoolNoSlot ? -1 : (int)pl.slot[b];
    split_body<DT, G, KH, true>(mem, window_w, knew, vnew, slot, q, ws_ml, ws_acc, Hkv, max_pages,
                                page_bytes, k, res_base, (int)pl.n_pages[b], (int)pl.n_res[b], S,
                                pl.gps, pl.max_splits, qscale, b * Hkv + h, split, table);
}

// Row bq = (sequence, query head) merges that sequence's S_b + W_b partials;
// D / (32 CPL) workgroups per row.
template <int PER, int CPL>
__global__ __launch_bounds__(kCombineThreads) void pool_combine_kernel(
    const float *__restrict__ ws_ml, const float *__restrict__ ws_acc, float *__restrict__ out,
    int Hq, int Hkv, const PoolPlan pl) {
    constexpr int kSlices = D / (32 * CPL);
    const int bq = blockIdx.x / kSlices;
    const int b = bq / Hq;
    const int n = (int)(pl.page_pref[b + 1] - pl.page_pref[b] + pl.win_pref[b + 1] -
                        pl.win_pref[b]) / Hkv;
    combine_body<PER, CPL>(ws_ml, ws_acc, out, n, pl.max_splits, bq, blockIdx.x % kSlices);
}

template <int PER, int CPL>
hipError_t launch_pool_combine(const Geometry &G, const float *ml, const float *acc, float *out,
                               const PoolPlan &pl, hipStream_t st) {
    hipLaunchKernelGGL((pool_combine_kernel<PER, CPL>), dim3(G.B * G.Hq * (D / (32 * CPL))),
                       dim3(kCombineThreads), 0, st, ml, acc, out, G.Hq, G.Hkv, pl);
    return hipGetLastError();
}

template <int DT, int G, int KH>
int pslots3() {
    static int cached = 0;
    if (cached) return cached;
    int per_cu = 0, dev = 0;
    hipDeviceProp_t prop;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pool_split_kernel<DT, G, KH>, 64,
                                                     0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        per_cu <= 0) {
        (void)hipGetLastError();
        return 2048;
    }
    cached = per_cu * prop.multiProcessorCount;
    return cached;
}

template <int DT, int G, int KH>
hipError_t plaunch3(const Geometry &Gm, uint8_t *mem, const int32_t *table, const uint16_t *kn,
                    const uint16_t *vn, const uint16_t *q, float *ml, float *acc,
                    const PoolPlan &pl, hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
    const uint32_t wgs = pl.page_pref[pl.n_seq] + pl.win_pref[pl.n_seq];
    if (wgs == 0) return hipSuccess;
    // with timing events: the dispatch's own start and end timestamps
    hipExtLaunchKernelGGL((pool_split_kernel<DT, G, KH>), dim3(wgs), dim3(64), 0, st, e0, e1, 0,
                          (const uint8_t *)mem, mem, kn, vn, q, ml, acc, table, Gm.Hkv,
                          Gm.max_pages, Gm.page_bytes, Gm.k, Gm.res_base, Gm.scale * kLog2e, pl);
    return hipGetLastError();
}

template <int DT, int G>
hipError_t plaunch2(const Geometry &Gm, uint8_t *mem, const int32_t *table, const uint16_t *kn,
                    const uint16_t *vn, const uint16_t *q, float *ml, float *acc,
                    const PoolPlan &pl, hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
    switch ((Gm.k + 31) / 32) {
        case 0: return plaunch3<DT, G, 0>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        case 1: return plaunch3<DT, G, 1>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        case 2: return plaunch3<DT, G, 2>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        case 3: return plaunch3<DT, G, 3>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        case 4: return plaunch3<DT, G, 4>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t plaunch1(const Geometry &Gm, uint8_t *mem, const int32_t *table, const uint16_t *kn,
                    const uint16_t *vn, const uint16_t *q, float *ml, float *acc,
                    const PoolPlan &pl, hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
    switch (Gm.g) {
        case 1: return plaunch2<DT, 1>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        case 2: return plaunch2<DT, 2>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        case 4: return plaunch2<DT, 4>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        case 8: return plaunch2<DT, 8>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        case 16: return plaunch2<DT, 16>(Gm, mem, table, kn, vn, q, ml, acc, pl, e0, e1, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, int G>
int pslots2(int k) {
    switch ((k + 31) / 32) {
        case 0: return pslots3<DT, G, 0>();
        case 1: return pslots3<DT, G, 1>();
        case 2: return pslots3<DT, G, 2>();
        case 3: return pslots3<DT, G, 3>();
        default: return pslots3<DT, G, 4>();
    }
}
template <int DT>
int pslots1(int g, int k) {
    switch (g) {
        case 1: return pslots2<DT, 1>(k);
        case 2: return pslots2<DT, 2>(k);
        case 4: return pslots2<DT, 4>(k);
        case 8: return pslots2<DT, 8>(k);
        default: return pslots2<DT, 16>(k);
    }
}

}  // namespace

int pool_decode_slots(const Geometry &G) {
    return G.dtype == F16 ? pslots1<F16>(G.g, G.k) : pslots1<BF16>(G.g, G.k);
}

hipError_t launch_pool_decode(const Geometry &G, uint8_t *mem, const int32_t *table,
                              const uint16_t *q, float *out, void *workspace, const PoolPlan &pl,
                              const uint16_t *kn, const uint16_t *vn, hipEvent_t ev_before,
                              hipEvent_t ev_after, hipStream_t st) {
    if (!kn || !vn) kn = vn = q;  // never dereferenced: every plan slot is kPoolNoSlot
    if (pl.max_splits > kMaxCombine) return hipErrorInvalidValue;
    float *ml = reinterpret_cast<float *>(workspace);
    float *acc = ml + (size_t)G.B * G.Hq * pl.max_splits * 2;
    hipError_t e =
        G.dtype == F16 ? plaunch1<F16>(G, mem, table, kn, vn, q, ml, acc, pl, ev_before, ev_after, st)
                       : plaunch1<BF16>(G, mem, table, kn, vn, q, ml, acc, pl, ev_before, ev_after, st);
    if (e != hipSuccess) return e;
    int max_n = 0;
    for (int b = 0; b < pl.n_seq; b++)
        max_n = std::max(max_n, (int)(pl.page_pref[b + 1] - pl.page_pref[b] + pl.win_pref[b + 1] -
                                      pl.win_pref[b]) / G.Hkv);
    const CombineShape cs = combine_shape(G.B * G.Hq, max_n);
    if (cs.cpl == 4)
        return cs.per == 8 ? launch_pool_combine<8, 4>(G, ml, acc, out, pl, st)
                           : launch_pool_combine<kCombinePerMax, 4>(G, ml, acc, out, pl, st);
    return cs.per == 8 ? launch_pool_combine<8, 1>(G, ml, acc, out, pl, st)
                       : launch_pool_combine<kCombinePerMax, 1>(G, ml, acc, out, pl, st);
}

}  // namespace kvq
