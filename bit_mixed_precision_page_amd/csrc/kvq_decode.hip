// kvq_decode.hip -- split-K GQA decode attention over the dense cache: the
// kernels that map a 1-D grid onto (unit, split), the combine kernel and the
// launchers.  The work itself is in kvq_decode_core.h.
#include <mutex>

#include "kvq_decode_core.h"
#include "kvq_quantize_core.h"

// Partials of kvq_decode_attention_noalloc: device memory that no call
// allocates.  Each GPU the library runs on holds its own copy until the
// process ends; every no-allocation call on that GPU shares it.
static __device__ __align__(256) uint8_t scratch[kvq::kStaticScratchBytes];

namespace kvq {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// 1-D grid of kDecodeWaves-wave workgroups: every page split of every
// (sequence, KV head) first, then the window splits, so the hardware places
// the long page workgroups evenly and the short window workgroups run as
// they drain.
//
// Counters of a graph-replayed step, in device memory:
//   dstate[0], dstate[1]  pages and window tokens at the start of the step;
//   dstate[3]             error flag (a token that found the cache full);
//   dstate[4], dstate[5]  pages and window tokens after the step's append,
//                         written by the split launch for the merge launch.
// A step starts with room in its window unless the cache is full: a window
// that a step fills is flushed into a page by that step's merge launch (the
// flush the next step would otherwise start with).  The new token takes
// window slot dstate[1]; with a full window (no free page was left) the step
// skips it and raises the flag.
__device__ __forceinline__ void step_state(int nr, int *slot, int *n_res, bool *room) {
    *room = nr < R;
    *slot = *room ? nr : -1;
    *n_res = *room ? nr + 1 : R;
}

// dstate != null: a step whose counters live in device memory, so that its
// launches have the same arguments at every step and can be replayed from a
// captured graph.  The kernel derives the step's state and covers the pages
// with page_splits splits of ceil(4 pages / (page_splits kDecodeWaves))
// groups per wave (empty runs and window waves past the last token write
// empty partials); its first thread records the counters after the append,
// which no other workgroup of this launch reads.
template <int DT, int G, int KH>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(waves_target(G, KH)))) void decode_split_kernel(
    const uint8_t *__restrict__ cache, uint8_t *__restrict__ window_w,
    const uint16_t *__restrict__ knew, const uint16_t *__restrict__ vnew, int slot,
    const uint16_t *__restrict__ q, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int Hkv, int max_pages, uint32_t page_bytes, int k,
    size_t res_base, int n_pages, int n_res, int page_splits, int gps, int win_splits, int max_splits,
    float qscale, int32_t *__restrict__ dstate) {
    if (dstate) {
        bool room;
        n_pages = dstate[0];
        step_state(dstate[1], &slot, &n_res, &room);
        gps = max(1, (4 * n_pages + page_splits * kDecodeWaves - 1) / (page_splits * kDecodeWaves));
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            dstate[4] = n_pages;
            dstate[5] = n_res;
            if (!room) dstate[3] = 1;
        }
    }
    const int n_units = gridDim.x / (page_splits + win_splits);
    int unit, split;
    dense_split_of(blockIdx.x, n_units, page_splits, win_splits, &unit, &split);
    split_body<DT, G, KH, false, kDecodeWaves>(cache, window_w, knew, vnew, slot, q, ws_ml, ws_acc, Hkv,
                                 max_pages, page_bytes, k, res_base, n_pages, n_res, page_splits,
                                 gps, max_splits, qscale, unit, split, nullptr);
}

// Device counters for graph-replayed steps.
__global__ void state_init_kernel(int32_t *dstate, int n_pages, int n_res) {
    for (int i = 0; i < kDeviceStateWords; i++) dstate[i] = 0;
    dstate[0] = n_pages;
    dstate[1] = n_res;
}

// D / (32 CPL) workgroups per output row.
template <int PER, int CPL>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float *__restrict__ ws_ml,
                                                                  const float *__restrict__ ws_acc,
                                                                  float *__restrict__ out, int n,
                                                                  int max_splits) {
    constexpr int kSlices = D / (32 * CPL);
    combine_body<PER, CPL>(ws_ml, ws_acc, out, n, max_splits, blockIdx.x / kSlices,
                           blockIdx.x % kSlices);
}

// Few splits per row: one wave per output row (sequence, query head).  Each
// lane issues every load of its row at once -- the n split statistics
// (the same address in every lane, one request per wave) and its two
// channels of each partial -- so a row costs one memory round trip, with no
// LDS and no barrier.
template <int NMAX>
__device__ __forceinline__ void combine_wave_body(const float *__restrict__ ws_ml,
                                                  const float *__restrict__ ws_acc,
                                                  float *__restrict__ out, int rows, int n,
                                                  int max_splits, int wg) {
    const int row = wg * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float2 *ml = reinterpret_cast<const float2 *>(ws_ml + (size_t)row * max_splits * 2);
    const float *a = ws_acc + (size_t)row * max_splits * D + 2 * lane;
    float2 st[NMAX], x[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; s++) {
        st[s] = s < n ? ml[s] : make_float2(-INFINITY, 0.0f);
        x[s] = s < n ? *reinterpret_cast<const float2 *>(a + (size_t)s * D) : make_float2(0.0f, 0.0f);
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NMAX; s++) M = fmaxf(M, st[s].x);
    float den = 0.0f, ax = 0.0f, ay = 0.0f;
#pragma unroll
    for (int s = 0; s < NMAX; s++) {
        const float w = s < n ? __builtin_amdgcn_exp2f(st[s].x - M) : 0.0f;
        den = fmaf(w, st[s].y, den);
        ax = fmaf(w, x[s].x, ax);
        ay = fmaf(w, x[s].y, ay);
    }
    *reinterpret_cast<float2 *>(out + (size_t)row * D + 2 * lane) =
        den > 0.0f ? make_float2(ax / den, ay / den) : make_float2(0.0f, 0.0f);
}
template <int NMAX>
__global__ __launch_bounds__(256) void combine_wave_kernel(const float *__restrict__ ws_ml,
                                                           const float *__restrict__ ws_acc,
                                                           float *__restrict__ out, int rows, int n,
                                                           int max_splits) {
    combine_wave_body<NMAX>(ws_ml, ws_acc, out, rows, n, max_splits, blockIdx.x);
}

// Merge launch of a graph-replayed step: workgroups [0, n_merge) merge the
// split partials exactly as the combine kernels do; workgroup n_merge + u
// flushes unit u's window into page dstate[4] when the step filled it and a
// page is free (the quantizer of the page launches).  Its first thread
// stores the counters the next step starts from; the other workgroups read
// only dstate[4], dstate[5], which the split launch wrote.
struct StepFlush {
    uint8_t *cache;
    size_t res_base;
    int max_pages, k;
    uint32_t page_bytes;
    const float *rel;  // [B][Hkv][D] or null
};
template <int DT>
__device__ __forceinline__ void step_flush(const int32_t *dstate, const StepFlush &f, int unit) {
    const int np = dstate[4], nr = dstate[5];
    if (nr != R || np >= f.max_pages) return;  // workgroup-uniform
    const uint16_t *kw = reinterpret_cast<const uint16_t *>(f.cache + f.res_base) +
                         (size_t)unit * 2 * R * D;
    uint8_t *pg = f.cache + ((size_t)unit * f.max_pages + np) * f.page_bytes;
    qz::quantize_page_body<DT>(pg, kw, kw + (size_t)R * D, f.k,
                               f.rel ? f.rel + (size_t)unit * D : nullptr);
}
__device__ __forceinline__ void step_advance(int32_t *dstate, int max_pages) {
    const int np = dstate[4], nr = dstate[5];
    const bool flush = nr == R && np < max_pages;
    dstate[0] = flush ? np + 1 : np;
    dstate[1] = flush ? 0 : nr;
}
static_assert(qz::kThreads == 256 && kCombineThreads == 256, "one workgroup shape for both roles");
template <int DT, int NMAX>
__global__ __launch_bounds__(256) void step_merge_wave_kernel(const float *__restrict__ ws_ml,
                                                              const float *__restrict__ ws_acc,
                                                              float *__restrict__ out, int rows,
                                                              int n, int max_splits, int n_merge,
                                                              int32_t *dstate, StepFlush f) {
    if (blockIdx.x == 0 && threadIdx.x == 0) step_advance(dstate, f.max_pages);
    if ((int)blockIdx.x >= n_merge) return step_flush<DT>(dstate, f, blockIdx.x - n_merge);
    combine_wave_body<NMAX>(ws_ml, ws_acc, out, rows, n, max_splits, blockIdx.x);
}
template <int DT, int PER, int CPL>
__global__ __launch_bounds__(kCombineThreads) void step_merge_kernel(const float *__restrict__ ws_ml,
                                                                     const float *__restrict__ ws_acc,
                                                                     float *__restrict__ out, int n,
                                                                     int max_splits, int n_merge,
                                                                     int32_t *dstate, StepFlush f) {
    constexpr int kSlices = D / (32 * CPL);
    if (blockIdx.x == 0 && threadIdx.x == 0) step_advance(dstate, f.max_pages);
    if ((int)blockIdx.x >= n_merge) return step_flush<DT>(dstate, f, blockIdx.x - n_merge);
    combine_body<PER, CPL>(ws_ml, ws_acc, out, n, max_splits, blockIdx.x / kSlices,
                           blockIdx.x % kSlices);
}

// Merge of the split partials; with a graph-replayed step (dstate) the
// merge launch also flushes a window the step filled and advances the
// counters (n_units more workgroups).
struct MergeArgs {
    int rows, n, max_splits, n_units;
    int32_t *dstate;
    StepFlush flush;
};
template <int NMAX>
hipError_t launch_combine_wave(int dtype, const MergeArgs &m, const float *ml, const float *acc,
                               float *out, hipStream_t st) {
    const int wgs = (m.rows + 3) / 4;
    if (!m.dstate)
        hipLaunchKernelGGL((combine_wave_kernel<NMAX>), dim3(wgs), dim3(256), 0, st, ml, acc, out,
                           m.rows, m.n, m.max_splits);
    else if (dtype == F16)
        hipLaunchKernelGGL((step_merge_wave_kernel<F16, NMAX>), dim3(wgs + m.n_units), dim3(256), 0,
                           st, ml, acc, out, m.rows, m.n, m.max_splits, wgs, m.dstate, m.flush);
    else
        hipLaunchKernelGGL((step_merge_wave_kernel<BF16, NMAX>), dim3(wgs + m.n_units), dim3(256), 0,
                           st, ml, acc, out, m.rows, m.n, m.max_splits, wgs, m.dstate, m.flush);
    return hipGetLastError();
}

template <int PER, int CPL>
hipError_t launch_combine(int dtype, const MergeArgs &m, const float *ml, const float *acc,
                          float *out, hipStream_t st) {
    const int wgs = m.rows * (D / (32 * CPL));
    if (!m.dstate)
        hipLaunchKernelGGL((combine_kernel<PER, CPL>), dim3(wgs), dim3(kCombineThreads), 0, st, ml,
                           acc, out, m.n, m.max_splits);
    else if (dtype == F16)
        hipLaunchKernelGGL((step_merge_kernel<F16, PER, CPL>), dim3(wgs + m.n_units),
                           dim3(kCombineThreads), 0, st, ml, acc, out, m.n, m.max_splits, wgs,
                           m.dstate, m.flush);
    else
        hipLaunchKernelGGL((step_merge_kernel<BF16, PER, CPL>), dim3(wgs + m.n_units),
                           dim3(kCombineThreads), 0, st, ml, acc, out, m.n, m.max_splits, wgs,
                           m.dstate, m.flush);
    return hipGetLastError();
}

// Resident waves of this instantiation on the whole device (occupancy API),
// cached; 2048 when no device answers (host-only use).
template <int DT, int G, int KH>
int slots3() {
    static int cached = 0;
    if (cached) return cached;
    int per_cu = 0, dev = 0;
    hipDeviceProp_t prop;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<DT, G, KH>,
                                                     64 * kDecodeWaves, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        per_cu <= 0) {
        (void)hipGetLastError();
        return 2048;
    }
    cached = per_cu * kDecodeWaves * prop.multiProcessorCount;
    return cached;
}

template <int DT, int G, int KH>
hipError_t launch3(const Geometry &Gm, uint8_t *cache, const uint16_t *kn, const uint16_t *vn,
                   int slot, const uint16_t *q, float *ml, float *acc, const DecodePlan &pl,
                   hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
    dim3 grid(pl.total_splits * Gm.Hkv * Gm.B);
    // with timing events: the dispatch's own start and end timestamps
    hipExtLaunchKernelGGL((decode_split_kernel<DT, G, KH>), grid, dim3(64 * kDecodeWaves), 0, st,
                          e0, e1, 0, (const uint8_t *)cache, cache, kn, vn, slot, q, ml, acc,
                          Gm.Hkv, Gm.max_pages, Gm.page_bytes, Gm.k, Gm.res_base, pl.n_pages,
                          pl.n_res, pl.page_splits, pl.groups_per_split,
                          pl.total_splits - pl.page_splits, pl.max_splits, Gm.scale * kLog2e,
                          pl.dstate);
    return hipGetLastError();
}

template <int DT, int G>
hipError_t launch2(const Geometry &Gm, uint8_t *cache, const uint16_t *kn, const uint16_t *vn,
                   int slot, const uint16_t *q, float *ml, float *acc, const DecodePlan &pl,
                   hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
    switch ((Gm.k + 31) / 32) {
        case 0: return launch3<DT, G, 0>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        case 1: return launch3<DT, G, 1>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        case 2: return launch3<DT, G, 2>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        case 3: return launch3<DT, G, 3>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        case 4: return launch3<DT, G, 4>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t launch1(const Geometry &Gm, uint8_t *cache, const uint16_t *kn, const uint16_t *vn,
                   int slot, const uint16_t *q, float *ml, float *acc, const DecodePlan &pl,
                   hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
    switch (Gm.g) {
        case 1: return launch2<DT, 1>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        case 2: return launch2<DT, 2>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        case 4: return launch2<DT, 4>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        case 8: return launch2<DT, 8>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
        case 16: return launch2<DT, 16>(Gm, cache, kn, vn, slot, q, ml, acc, pl, e0, e1, st);
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

// Device address of the current device's `scratch`, looked up once per device
// (with that device current) and kept; the host-side name of the array is
// only a stand-in and is never passed to a kernel.
hipError_t static_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return hipSuccess;
}

int decode_slots(const Geometry &G) {
    return G.dtype == F16 ? slots1<F16>(G.g, G.k) : slots1<BF16>(G.g, G.k);
}

size_t decode_workspace_bytes(const Geometry &G, int max_splits) {
    size_t rows = (size_t)G.B * G.Hq * max_splits;
    return rows * 2 * sizeof(float) + rows * D * sizeof(float);
}

hipError_t launch_state_init(int32_t *dstate, int n_pages, int n_res, hipStream_t st) {
    hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(1), 0, st, dstate, n_pages, n_res);
    return hipGetLastError();
}

hipError_t launch_decode(const Geometry &G, uint8_t *cache, const uint16_t *q,
                         float *out, void *workspace, const DecodePlan &pl,
                         const uint16_t *kn, const uint16_t *vn, int slot,
                         hipEvent_t ev_before, hipEvent_t ev_after, hipStream_t st) {
    if (slot < 0) kn = vn = q;  // never dereferenced: no window token equals slot -1
    if (pl.total_splits > kMaxCombine) return hipErrorInvalidValue;  // before any launch
    float *ml = reinterpret_cast<float *>(workspace);
    float *acc = ml + (size_t)G.B * G.Hq * pl.max_splits * 2;
    const hipError_t e =
        G.dtype == F16 ? launch1<F16>(G, cache, kn, vn, slot, q, ml, acc, pl, ev_before, ev_after, st)
                       : launch1<BF16>(G, cache, kn, vn, slot, q, ml, acc, pl, ev_before, ev_after, st);
    if (e != hipSuccess) return e;
    MergeArgs m{};
    m.rows = G.B * G.Hq;
    m.n = pl.total_splits;
    m.max_splits = pl.max_splits;
    m.n_units = G.B * G.Hkv;
    m.dstate = pl.dstate;
    m.flush = StepFlush{cache, G.res_base, G.max_pages, G.k, G.page_bytes, pl.rel};
    const int dt = G.dtype;
    if (m.n <= 16) return launch_combine_wave<16>(dt, m, ml, acc, out, st);
    if (m.n <= 32) return launch_combine_wave<32>(dt, m, ml, acc, out, st);
    const CombineShape cs = combine_shape(m.rows, m.n);
    if (cs.cpl == 4)
        return cs.per == 8 ? launch_combine<8, 4>(dt, m, ml, acc, out, st)
                           : launch_combine<kCombinePerMax, 4>(dt, m, ml, acc, out, st);
    return cs.per == 8 ? launch_combine<8, 1>(dt, m, ml, acc, out, st)
                       : launch_combine<kCombinePerMax, 1>(dt, m, ml, acc, out, st);
}

}  // namespace kvq
