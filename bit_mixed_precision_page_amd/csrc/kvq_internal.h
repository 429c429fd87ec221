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
// Same, reading the counters from device memory ({pages, window tokens, ..}):
// does nothing unless the window is full and a page is free.
hipError_t launch_flush_window_device(const Geometry &G, uint8_t *cache, const int32_t *dstate,
                                      const float *rel, hipStream_t stream);
// dstate <- {n_pages, n_res, 0, 0}
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

struct DecodePlan {
    int n_pages, n_res;
    int page_splits;      // splits over the 32-token page groups (0 when n_pages == 0)
    int groups_per_split;
    int total_splits;     // page_splits + ceil(n_res / 32) window splits
    int max_splits;       // workspace stride (splits per (b, hq))
    int32_t *dstate;      // non-null: counters in device memory (graph-replayable step);
                          // then total_splits = page_splits + R / 32
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
