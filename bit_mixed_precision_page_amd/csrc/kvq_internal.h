// kvq_internal.h -- layout constants, device helpers and kernel launchers of
// the 2-bit mixed-precision KV cache library (gfx950).  Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace kvq {

constexpr int D = 128;   // head dimension
constexpr int P = 128;   // tokens per page
constexpr int GK = 32;   // tokens per Key group (one channel)
constexpr int GV = 32;   // channels per Value group (one token)
constexpr int R = 128;   // window tokens
constexpr int F16 = 0, BF16 = 1;

// Page segments (Kitty abstract: page-centric layout, Key page as two
// uniform 2-bit planes).  Every segment is 16-byte aligned because k is a
// multiple of 16.
struct PageLayout {
    uint32_t klo, khi, ks, kz, kidx, vc, vs, vz, bytes;
};

__host__ __device__ constexpr PageLayout page_layout(int k) {
    PageLayout L{};
    uint32_t o = 0;
    L.klo = o;  o += P * D / 4;
    L.khi = o;  o += P * k / 4;
    L.ks = o;   o += (P / GK) * D * 2;
    L.kz = o;   o += (P / GK) * D * 2;
    L.kidx = o; o += (uint32_t)((k + 15) / 16 * 16);
    L.vc = o;   o += P * D / 4;
    L.vs = o;   o += (D / GV) * P * 2;
    L.vz = o;   o += (D / GV) * P * 2;
    L.bytes = o;
    return L;
}

// Geometry of one cache, shared by the launchers.
struct Geometry {
    int B, Hq, Hkv, g, k, max_pages, dtype;
    uint32_t page_bytes;
    size_t res_base;  // byte offset of the window region
    float scale;      // softmax scale
};

__host__ __device__ inline size_t page_off(const Geometry &G, int unit, int page) {
    return ((size_t)unit * G.max_pages + page) * G.page_bytes;
}
__host__ __device__ inline size_t res_k_off(const Geometry &G, int unit) {
    return G.res_base + (size_t)unit * 2 * R * D * 2;
}
__host__ __device__ inline size_t res_v_off(const Geometry &G, int unit) {
    return res_k_off(G, unit) + (size_t)R * D * 2;
}

// Launchers (defined in the .hip files).  All asynchronous on `stream`.
// Quantize `n_new` pages per unit: the source of page p of unit u starts at
// element src + u * src_unit_stride + p * P * D of k_src / v_src ([P][D] rows
// of D contiguous elements); destinations are pages first_page + p.  rel:
// [B][Hkv][D] channel relevance (query-aware ranking) or null (magnitude).
hipError_t launch_quantize_pages(const Geometry &G, uint8_t *cache, const uint16_t *k_src,
                                 const uint16_t *v_src, size_t src_unit_stride,
                                 int first_page, int n_new, const float *rel,
                                 hipStream_t stream);
// Same, with each unit's window as the source (one page per unit).
hipError_t launch_flush_window(const Geometry &G, uint8_t *cache, int page, const float *rel,
                               hipStream_t stream);
// Words of a graph-replayed step's device counters, and their initial
// values: dstate <- {n_pages, n_res, 0, ...}.
constexpr int kDeviceStateWords = 8;
hipError_t launch_state_init(int32_t *dstate, int n_pages, int n_res, hipStream_t stream);
// rel [B][Hkv][D] = sum over each KV head's query heads of |q| (q [B][Hq][D]).
hipError_t launch_query_relevance(int dtype, const uint16_t *q, float *rel, int B, int Hq,
                                  int Hkv, hipStream_t stream);
// Copy one token per unit into window slot `slot`.
hipError_t launch_append(const Geometry &G, uint8_t *cache, const uint16_t *k,
                         const uint16_t *v, int slot, hipStream_t stream);
// Quantize arbitrary groups (inspection entry point).
hipError_t launch_quantize_groups(int dtype, int L, const uint16_t *x, int n_groups,
                                  int group_len, uint16_t *s, uint16_t *z, uint8_t *codes,
                                  hipStream_t stream);

// Splits (page + window) one combine workgroup merges per output row.
constexpr int kMaxCombineSplits = 272;

// Work of wave wv (of nw) of split `split` of one (sequence, KV head) unit
// in a decode launch: a page split (split < page_splits) streams the unit's
// Key groups [g0, g1) (four 32-token groups per page); a window split covers
// window tokens [t0, t1) (t1 <= t0: none; its loads then read token
// n_res - 1).  The decode kernels and the host-side extent check
// (kvq_check_decode_plan) both take their indices from here.
struct WaveWork {
    bool window;
    int g0, g1, t0, t1;
};
__host__ __device__ inline WaveWork wave_work(int split, int wv, int nw, int page_splits, int gps,
                                              int n_pages, int n_res) {
    WaveWork w{};
    if (split >= page_splits) {
        w.window = true;
        w.t0 = 32 * ((split - page_splits) * nw + wv);
        w.t1 = n_res < w.t0 + 32 ? n_res : w.t0 + 32;
    } else {
        w.g0 = (split * nw + wv) * gps;
        w.g1 = 4 * n_pages < w.g0 + gps ? 4 * n_pages : w.g0 + gps;
    }
    return w;
}
// Workgroup x of the dense decode kernel's 1-D grid: every page split of
// every unit first (unit-major), then the window splits.
__host__ __device__ inline void dense_split_of(int x, int n_units, int page_splits, int win_splits,
                                               int *unit, int *split) {
    if (x < page_splits * n_units) {
        *unit = x / page_splits;
        *split = x % page_splits;
    } else {
        const int l = x - page_splits * n_units;
        *unit = l / win_splits;
        *split = page_splits + l % win_splits;
    }
}
// Partial (m, l, acc) slot of query row bq = b Hq + hq, split `split`.
__host__ __device__ inline size_t partial_index(size_t bq, int max_splits, int split) {
    return bq * (size_t)max_splits + (size_t)split;
}

struct DecodePlan {
    int n_pages, n_res;
    int page_splits;      // splits over the 32-token page groups (0 when n_pages == 0)
    int groups_per_split;
    int total_splits;     // page_splits + ceil(n_res / 32) window splits
    int max_splits;       // workspace stride (splits per (b, hq))
    int32_t *dstate;      // non-null: counters in device memory (graph-replayable step);
                          // then total_splits = page_splits + R / 32
    const float *rel;     // with dstate: channel relevance of the window flush of the
                          // merge launch ([B][Hkv][D]), or null
};
size_t decode_workspace_bytes(const Geometry &G, int max_splits);

// Query chunks the column sums of the cumulative scores are split over.
constexpr int kColsumChunks = 16;
// Short sequences give the attention kernel too few workgroups for the chip:
// then the keys of each row block are split into up to kPrefillMaxKeySplits
// chunks of kbc 32-key blocks, each chunk a workgroup writing unnormalized
// partials that a merge kernel combines.  Returns the chunk count (1: no
// split, kbc = every block).
constexpr int kPrefillSplitWgs = 768;     // three attention workgroups per CU
constexpr int kPrefillMaxKeySplits = 4;
// cap > 0 bounds the chunk count (a caller's override; 0 = automatic).
inline int prefill_key_splits(int T, int Hq, int Hkv, int *kbc, int cap = 0) {
    const int g = Hq / Hkv, hw = g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1;
    const int qr = 128 / hw, nb = (T + 31) / 32;
    const long wgs = (long)(Hq / hw) * ((T + qr - 1) / qr);
    int s = 1;
    if (wgs < kPrefillSplitWgs)
        s = (int)std::min<long>(kPrefillMaxKeySplits, (kPrefillSplitWgs + wgs - 1) / wgs);
    if (cap > 0) s = std::min(s, cap);
    *kbc = (nb + s - 1) / s;
    return (nb + *kbc - 1) / *kbc;
}
// Prefill of one sequence: causal attention with cumulative attention scores,
// heavy-hitter + recent token selection and the gather of the kept rows.
struct PrefillArgs {
    int T, T32, Hq, Hkv, heavy, recent, n_keep;
    float scale;
    const uint16_t *q, *k, *v;  // [Hq][T][D], [Hkv][T][D], [Hkv][T][D]
    uint16_t *vt;               // workspace: [Hkv][T32 / 32][D][32] transposed Values
    float *lse;                 // workspace: [Hq][T] log2 of each row's softmax denominator
    float *part;                // workspace: [Hkv][kColsumChunks][T] partial column sums
    float *out, *score;         // [Hq][T][D], [Hkv][T]
    int32_t *keep;              // [Hkv][n_keep]
    uint16_t *k_sel, *v_sel;    // [Hkv][n_keep][D], or null
    int nsplit, kbc;            // key chunks per row block, 32-key blocks per chunk
    float *pml, *pacc;          // workspace when nsplit > 1: [Hq][T][nsplit] (m, l), (.., D) acc
    hipEvent_t ev_before, ev_after;  // optional, around the attention kernel
};
hipError_t launch_prefill(int dtype, const PrefillArgs &a, hipStream_t stream);
// Waves per workgroup of the dense decode kernel: each wave streams its own
// run of groups (or 32 window tokens) and the workgroup merges the waves'
// partials in LDS, so one split = kDecodeWaves runs.
constexpr int kDecodeWaves = 4;
// Waves of the decode kernel the device holds at once (2048 without a device).
int decode_slots(const Geometry &G);
// knew, vnew ([B][Hkv][D]) and slot >= 0: the newest window token (slot) is
// read from knew / vnew and written into the window by the kernel itself (a
// fused append); slot = -1: the window is read as it is.
// Bandwidth probe: mode 0 streams `bytes` of src (a 4-byte sink in dst),
// mode 1 copies them to dst.
hipError_t launch_probe(int mode, const void *src, void *dst, size_t bytes, hipStream_t stream);
// Bytes of the static partials buffer of the no-allocation decode call, and
// its device address on the current device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void **ptr);
hipError_t launch_decode(const Geometry &G, uint8_t *cache, const uint16_t *q,
                         float *out, void *workspace, const DecodePlan &plan,
                         const uint16_t *knew, const uint16_t *vnew, int slot,
                         hipEvent_t ev_before, hipEvent_t ev_after, hipStream_t stream);

// ---------------------------------------------------------------------------
// Block pool (variable-length batches).  A block holds the Hkv pages of one
// 128-token span of one sequence; sequence b's page p is block
// table[b * max_pages + p].  Per-launch lists travel by value in the kernel
// arguments (no host-to-device copies): at most kPoolMaxSeqs entries.
constexpr int kPoolMaxSeqs = 256;
constexpr int kPoolNoSlot = 255;

// Pages to quantize into pool blocks: entry e writes block[e] (all KV heads),
// records it at table[tslot[e]], and reads its rows at element
// src[e] * src_e_stride + h * src_h_stride of the sources.
struct PoolPages {
    int n;
    int32_t block[kPoolMaxSeqs];
    int32_t tslot[kPoolMaxSeqs];
    int32_t src[kPoolMaxSeqs];
};
// Window slot of the token each sequence takes (kPoolNoSlot: none).
struct PoolSlots {
    uint8_t slot[kPoolMaxSeqs];
};
// Decode work of a variable-length batch: sequence b owns Hkv * S_b page-split
// workgroups [page_pref[b], page_pref[b + 1]) and Hkv * W_b window workgroups
// [page_wgs + win_pref[b], page_wgs + win_pref[b + 1]), S_b = ceil(4 n_pages / gps),
// W_b = ceil(n_res / 32).
struct PoolPlan {
    int n_seq, page_wgs, gps, max_splits;
    uint32_t page_pref[kPoolMaxSeqs + 1];
    uint16_t win_pref[kPoolMaxSeqs + 1];
    uint16_t n_pages[kPoolMaxSeqs];
    uint8_t n_res[kPoolMaxSeqs];
    uint8_t slot[kPoolMaxSeqs];  // fused append: window slot of the new token, or kPoolNoSlot
};
// Last index b in [0, n) with pref[b] <= x (pref ascending, pref[n] > x).
template <typename T>
__host__ __device__ inline int pool_seq_of(const T *pref, int n, uint32_t x) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((uint32_t)pref[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}
// Workgroup x of the pool decode kernel's grid -> (sequence b, KV head h,
// split, page splits S of that sequence).
__host__ __device__ inline void pool_split_of(const PoolPlan &pl, int Hkv, uint32_t x, int *b,
                                              int *h, int *split, int *S) {
    if (x < (uint32_t)pl.page_wgs) {
        *b = pool_seq_of(pl.page_pref, pl.n_seq, x);
        *S = (int)(pl.page_pref[*b + 1] - pl.page_pref[*b]) / Hkv;
        const int l = (int)(x - pl.page_pref[*b]);
        *h = l / *S;
        *split = l % *S;
    } else {
        const uint32_t y = x - (uint32_t)pl.page_wgs;
        *b = pool_seq_of(pl.win_pref, pl.n_seq, y);
        *S = (int)(pl.page_pref[*b + 1] - pl.page_pref[*b]) / Hkv;
        const int W = (int)(pl.win_pref[*b + 1] - pl.win_pref[*b]) / Hkv;
        const int l = (int)(y - pl.win_pref[*b]);
        *h = l / W;
        *split = *S + l % W;
    }
}

// G describes the pool: B = sequence slots, max_pages = pages per sequence,
// res_base = byte offset of the windows ([B][Hkv][K | V][R][D]).
hipError_t launch_pool_pages(const Geometry &G, uint8_t *pool, int32_t *table,
                             const uint16_t *k_src, const uint16_t *v_src, size_t src_h_stride,
                             size_t src_e_stride, const PoolPages &pp, const float *rel,
                             hipStream_t stream);
hipError_t launch_pool_append(const Geometry &G, uint8_t *mem, const uint16_t *k,
                              const uint16_t *v, const PoolSlots &ps, hipStream_t stream);
hipError_t launch_pool_window_fill(const Geometry &G, uint8_t *mem, const uint16_t *k,
                                   const uint16_t *v, int seq, int n_tokens, int first, int tail,
                                   hipStream_t stream);
int pool_decode_slots(const Geometry &G);
// knew / vnew ([B][Hkv][D]) are read for the sequences whose plan slot is set.
hipError_t launch_pool_decode(const Geometry &G, uint8_t *mem, const int32_t *table,
                              const uint16_t *q, float *out, void *workspace, const PoolPlan &pl,
                              const uint16_t *knew, const uint16_t *vnew, hipEvent_t ev_before,
                              hipEvent_t ev_after, hipStream_t stream);

}  // namespace kvq
