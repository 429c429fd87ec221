// kvq_decode.hip -- split-K GQA decode attention over the dense cache: the
// kernels that map a 1-D grid onto (unit, split), the combine kernel and the
// launchers.  The work itself is in kvq_decode_core.h.
#include "kvq_decode_core.h"

namespace kvq {
namespace {

// 1-D grid of kDecodeWaves-wave workgroups: every page split of every
// (sequence, KV head) first, then the window splits, so the hardware places
// the long page workgroups evenly and the short window workgroups run as
// they drain.
//
// dstate != null: a step whose counters live in device memory (dstate =
// {pages, window tokens, finished-workgroup count, error}), so that its
// launches have the same arguments at every step and can be replayed from a
// captured graph.  The kernel derives the step's state (a full window was
// flushed by the preceding quantize launch; the new token takes the next
// window slot), covers the pages with page_splits splits of
// ceil(4 pages / (page_splits kDecodeWaves)) groups per wave (empty runs and
// window waves past the
// last token write empty partials) and the last workgroup to finish stores
// the new counters.
template <int DT, int G, int KH>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(waves_target(G, KH)))) void decode_split_kernel(
    const uint8_t *__restrict__ cache, uint8_t *__restrict__ window_w,
    const uint16_t *__restrict__ knew, const uint16_t *__restrict__ vnew, int slot,
    const uint16_t *__restrict__ q, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int Hkv, int max_pages, uint32_t page_bytes, int k,
    size_t res_base, int n_pages, int n_res, int page_splits, int gps, int win_splits, int max_splits,
    float qscale, int32_t *__restrict__ dstate) {
    bool room = true;
    if (dstate) {
        const int np = dstate[0], nr = dstate[1];
        const bool full = nr == R;
        room = !full || np < max_pages;
        n_pages = full && room ? np + 1 : np;
        n_res = full ? (room ? 1 : R) : nr + 1;
        slot = room ? n_res - 1 : -1;
        gps = max(1, (4 * n_pages + page_splits * kDecodeWaves - 1) / (page_splits * kDecodeWaves));
    }
    const int n_units = gridDim.x / (page_splits + win_splits);
    int unit, split;
    if ((int)blockIdx.x < page_splits * n_units) {
        unit = blockIdx.x / page_splits;
        split = blockIdx.x % page_splits;
    } else {
        const int l = blockIdx.x - page_splits * n_units;
        unit = l / win_splits;
        split = page_splits + l % win_splits;
    }
    split_body<DT, G, KH, false, kDecodeWaves>(cache, window_w, knew, vnew, slot, q, ws_ml, ws_acc, Hkv,
                                 max_pages, page_bytes, k, res_base, n_pages, n_res, page_splits,
                                 gps, max_splits, qscale, unit, split, nullptr);
    if (dstate && threadIdx.x == 0) {
        // every other workgroup has finished (and read dstate at its start)
        // when the count reaches the grid size
        if (atomicAdd(reinterpret_cast<unsigned *>(dstate + 2), 1u) == gridDim.x - 1) {
            dstate[0] = n_pages;
            dstate[1] = n_res;
            dstate[2] = 0;
            if (!room) dstate[3] = 1;
        }
    }
}

// Device counters for graph-replayed steps.
__global__ void state_init_kernel(int32_t *dstate, int n_pages, int n_res) {
    dstate[0] = n_pages;
    dstate[1] = n_res;
    dstate[2] = 0;
    dstate[3] = 0;
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
__global__ __launch_bounds__(256) void combine_wave_kernel(const float *__restrict__ ws_ml,
                                                           const float *__restrict__ ws_acc,
                                                           float *__restrict__ out, int rows, int n,
                                                           int max_splits) {
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
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
hipError_t launch_combine_wave(int rows, const float *ml, const float *acc, float *out, int n,
                               int max_splits, hipStream_t st) {
    hipLaunchKernelGGL((combine_wave_kernel<NMAX>), dim3((rows + 3) / 4), dim3(256), 0, st, ml, acc,
                       out, rows, n, max_splits);
    return hipGetLastError();
}

template <int PER, int CPL>
hipError_t launch_combine(int rows, const float *ml, const float *acc, float *out, int n,
                          int max_splits, hipStream_t st) {
    hipLaunchKernelGGL((combine_kernel<PER, CPL>), dim3(rows * (D / (32 * CPL))),
                       dim3(kCombineThreads), 0, st, ml, acc, out, n, max_splits);
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
    float *ml = reinterpret_cast<float *>(workspace);
    float *acc = ml + (size_t)G.B * G.Hq * pl.max_splits * 2;
    const hipError_t e =
        G.dtype == F16 ? launch1<F16>(G, cache, kn, vn, slot, q, ml, acc, pl, ev_before, ev_after, st)
                       : launch1<BF16>(G, cache, kn, vn, slot, q, ml, acc, pl, ev_before, ev_after, st);
    if (e != hipSuccess) return e;
    if (pl.total_splits > kMaxCombine) return hipErrorInvalidValue;
    const int rows = G.B * G.Hq;
    if (pl.total_splits <= 16)
        return launch_combine_wave<16>(rows, ml, acc, out, pl.total_splits, pl.max_splits, st);
    if (pl.total_splits <= 32)
        return launch_combine_wave<32>(rows, ml, acc, out, pl.total_splits, pl.max_splits, st);
    const CombineShape cs = combine_shape(rows, pl.total_splits);
    if (cs.cpl == 4)
        return cs.per == 8 ? launch_combine<8, 4>(rows, ml, acc, out, pl.total_splits, pl.max_splits, st)
                           : launch_combine<kCombinePerMax, 4>(rows, ml, acc, out, pl.total_splits, pl.max_splits, st);
    return cs.per == 8 ? launch_combine<8, 1>(rows, ml, acc, out, pl.total_splits, pl.max_splits, st)
                       : launch_combine<kCombinePerMax, 1>(rows, ml, acc, out, pl.total_splits, pl.max_splits, st);
}

}  // namespace kvq
