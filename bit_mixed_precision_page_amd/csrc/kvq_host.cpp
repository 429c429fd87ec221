// kvq_host.cpp -- the C ABI of include/kvq.h: configuration checks, cache
// layout and counters, decode planning and kernel launches.  Never allocates
// or frees device memory and never synchronizes; every check happens before
// any launch so a failed call leaves the cache unchanged.
#include "../../include/kvq.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <new>
#include <vector>

#include "kvq_internal.h"

struct kvq_cache {
    kvq::Geometry G;
    uint8_t *mem;
    size_t bytes;
    int32_t n_pages;
    int32_t n_res;
    int32_t splits_override;  // 0 = automatic
    const float *rel;         // query-aware channel relevance [B][Hkv][D], or null
    hipEvent_t ev_before, ev_after;
};

// Block pool: host state of every sequence slot and the free list.
struct kvq_pool {
    kvq::Geometry G;  // B = slots, max_pages = pages per sequence, res_base = windows
    uint8_t *mem;
    size_t bytes;
    size_t table_off;
    int32_t n_blocks;
    std::vector<uint8_t> live;
    std::vector<int32_t> n_pages, n_res;
    std::vector<std::vector<int32_t>> blocks;
    std::vector<int32_t> free_list;  // back() is handed out next
    const float *rel;                // query-aware channel relevance [B][Hkv][D], or null
    hipEvent_t ev_before, ev_after;
};

namespace {

static_assert(kvq::kDeviceStateWords == KVQ_DEVICE_STATE_WORDS, "device state size");
constexpr int kMaxSplits = 256;  // page splits per (sequence, KV head)
constexpr int kRoundGroups = 32;  // groups per split when one round of waves cannot hold every unit

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_config(const kvq_config *c) {
    if (!c) return KVQ_EINVAL;
    if (c->batch < 1 || c->num_kv_heads < 1 || c->num_q_heads < 1) return KVQ_EINVAL;
    if (c->num_q_heads % c->num_kv_heads) return KVQ_EINVAL;
    int g = c->num_q_heads / c->num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return KVQ_EINVAL;
    if (c->head_dim != kvq::D || c->page_tokens != kvq::P || c->key_group_tokens != kvq::GK ||
        c->value_group_channels != kvq::GV || c->residual_tokens != kvq::R)
        return KVQ_EINVAL;
    if (c->boost_channels < 0 || c->boost_channels > kvq::D || c->boost_channels % 16)
        return KVQ_EINVAL;
    if (c->max_pages < 1 || c->max_pages > (1 << 24)) return KVQ_EINVAL;
    if (c->dtype != KVQ_F16 && c->dtype != KVQ_BF16) return KVQ_EINVAL;
    if (!std::isfinite(c->softmax_scale)) return KVQ_EINVAL;
    // the cache must be addressable with 64-bit offsets and < 2^31 units
    if ((int64_t)c->batch * c->num_kv_heads > (1 << 30)) return KVQ_EINVAL;
    return KVQ_OK;
}

kvq::Geometry geometry_of(const kvq_config *c) {
    kvq::Geometry G{};
    G.B = c->batch;
    G.Hq = c->num_q_heads;
    G.Hkv = c->num_kv_heads;
    G.g = c->num_q_heads / c->num_kv_heads;
    G.k = c->boost_channels;
    G.max_pages = c->max_pages;
    G.dtype = c->dtype;
    G.page_bytes = kvq::page_layout(G.k).bytes;
    G.res_base = (size_t)G.B * G.Hkv * G.max_pages * G.page_bytes;
    G.scale = c->softmax_scale > 0.0f ? c->softmax_scale : 1.0f / std::sqrt((float)kvq::D);
    return G;
}

size_t cache_bytes_of(const kvq::Geometry &G) {
    return G.res_base + (size_t)G.B * G.Hkv * 2 * kvq::R * kvq::D * 2;
}

int max_splits_of(const kvq::Geometry &G) {
    // page splits (at most one per 32-token group) + window splits (32 window
    // tokens per split)
    return std::min(4 * G.max_pages, kMaxSplits) + kvq::R / 32;
}

// Decode plan for the cache's pages and n_res window tokens (the host
// counter, or one more for a fused step whose token is not yet counted).
kvq::DecodePlan plan_of(const kvq_cache *c, int n_res, int slots = 0) {
    kvq::DecodePlan pl{};
    pl.n_pages = c->n_pages;
    pl.n_res = n_res;
    pl.max_splits = max_splits_of(c->G);
    if (c->n_pages > 0) {
        constexpr int NW = kvq::kDecodeWaves;
        const int groups = 4 * c->n_pages;
        int S;  // page splits (workgroups of NW waves, one run of groups each)
        if (c->splits_override > 0) {
            S = c->splits_override;
        } else {
            // One round of resident waves (occupancy of this kernel instance
            // x compute units) of page runs with equal groups per run; the
            // short window splits follow as the page workgroups drain (a
            // measured 2-3 % faster than sharing the round with them, and the
            // split count does not depend on the window length).  When the
            // units alone fill more than a round, runs of about kRoundGroups
            // groups fill several rounds and the hardware's dispatch balances
            // them.
            const int units = c->G.B * c->G.Hkv;
            const int per_unit = (slots > 0 ? slots : kvq::decode_slots(c->G)) / units;
            S = per_unit >= NW ? per_unit / NW
                               : (groups + kRoundGroups * NW - 1) / (kRoundGroups * NW);
        }
        S = std::max(1, std::min(S, std::min((groups + NW - 1) / NW, kMaxSplits)));
        pl.groups_per_split = (groups + S * NW - 1) / (S * NW);  // per wave
        pl.page_splits = (groups + pl.groups_per_split * NW - 1) / (pl.groups_per_split * NW);
    }
    pl.total_splits = pl.page_splits + (n_res + 32 * kvq::kDecodeWaves - 1) / (32 * kvq::kDecodeWaves);
    return pl;
}
kvq::DecodePlan plan_of(const kvq_cache *c) { return plan_of(c, c->n_res); }

// Plan of the graph-replayable step: page splits fixed for every replay (the
// override, or one round of resident waves sized for the host counters at
// this call; at least one, at most one wave per group of one more page than
// the cache holds now); the groups per wave follow on the device from the
// counters of each replay.
kvq::DecodePlan device_step_plan(const kvq_cache *c, int slots = 0) {
    constexpr int NW = kvq::kDecodeWaves;
    const int cap = std::min(kMaxSplits, (4 * std::min(c->G.max_pages, c->n_pages + 1) + NW - 1) / NW);
    int S;
    if (c->splits_override > 0) {
        S = c->splits_override;
    } else {
        const int units = c->G.B * c->G.Hkv;
        const int per_unit = (slots > 0 ? slots : kvq::decode_slots(c->G)) / units;
        S = per_unit >= NW ? per_unit / NW
                           : (4 * (c->n_pages + 1) + kRoundGroups * NW - 1) / (kRoundGroups * NW);
    }
    kvq::DecodePlan pl{};
    pl.page_splits = std::max(1, std::min(S, cap));
    pl.groups_per_split = 1;  // derived on the device from the counters
    pl.total_splits = pl.page_splits + (kvq::R + 32 * NW - 1) / (32 * NW);
    pl.max_splits = max_splits_of(c->G);
    return pl;
}

// The groups per wave a graph-replayed step derives on the device for
// n_pages pages (the same expression as the kernel's).
int device_step_gps(const kvq::DecodePlan &pl, int n_pages) {
    constexpr int NW = kvq::kDecodeWaves;
    return std::max(1, (4 * n_pages + pl.page_splits * NW - 1) / (pl.page_splits * NW));
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_EHIP; }

// ------------------------------------------------ host-side extent check ----
// Every workgroup and wave of a decode launch, walked with the kernels' own
// index helpers (kvq_internal.h): the byte ranges each wave reads and each
// split's partial slot must lie inside the cache and the workspace, every Key
// group and window token of a unit must be read by exactly one wave, and the
// split count must fit the combine kernel.  Out-of-range buffer loads on the
// device read zeros instead of faulting, so this is where an offset mistake
// in a plan shows.
struct PlanCheck {
    char *msg;
    size_t len;
    int fail(const char *what, long a, long b, long c2) {
        if (msg && len) snprintf(msg, len, "%s (%ld, %ld, %ld)", what, a, b, c2);
        return KVQ_EINVAL;
    }
};

bool inside(size_t off, size_t n, size_t lo, size_t hi) { return off >= lo && n <= hi - off && off <= hi; }

// One unit's work at (n_pages, n_res) under a split plan; `page_at` maps a
// page index to its byte offset, `win_off` is the unit's window K offset.
template <class PageAt>
int check_unit(PlanCheck &pc, const kvq::Geometry &G, int unit, int n_pages, int n_res,
               int page_splits, int win_splits, int gps, int nw, int max_splits,
               size_t pages_lo, size_t pages_hi, size_t win_off, size_t win_hi, size_t ws_bytes,
               PageAt page_at, std::vector<uint8_t> &seen_g, std::vector<uint8_t> &seen_t) {
    seen_g.assign((size_t)4 * n_pages, 0);
    seen_t.assign((size_t)n_res, 0);
    const size_t rows = (size_t)G.B * G.Hq;
    const size_t ml_bytes = rows * max_splits * 2 * sizeof(float);
    const int b = unit / G.Hkv, h = unit % G.Hkv;
    for (int split = 0; split < page_splits + win_splits; split++) {
        if (split >= max_splits) return pc.fail("split beyond the workspace stride", unit, split, max_splits);
        for (int hh = 0; hh < G.g; hh++) {
            const size_t bq = (size_t)b * G.Hq + (size_t)h * G.g + hh;
            const size_t pi = kvq::partial_index(bq, max_splits, split);
            if (pi >= rows * max_splits || !inside(ml_bytes + pi * kvq::D * 4, kvq::D * 4, 0, ws_bytes) ||
                !inside(pi * 8, 8, 0, ml_bytes))
                return pc.fail("partial outside the workspace", unit, split, hh);
        }
        for (int wv = 0; wv < nw; wv++) {
            const kvq::WaveWork w = kvq::wave_work(split, wv, nw, page_splits, gps, n_pages, n_res);
            if (w.window) {
                if (split < page_splits) return pc.fail("window work in a page split", unit, split, wv);
                if (n_res < 1) return pc.fail("window split without window tokens", unit, split, wv);
                for (int t = w.t0; t < w.t1; t++) {
                    if (t < 0 || t >= n_res) return pc.fail("window token out of range", unit, t, n_res);
                    if (seen_t[t]++) return pc.fail("window token read twice", unit, t, split);
                }
                // loads of a wave past the last token read token n_res - 1
                const int tmax = w.t1 > w.t0 ? w.t1 - 1 : n_res - 1;
                const size_t kb = win_off + (size_t)tmax * kvq::D * 2;
                const size_t vb = win_off + (size_t)kvq::R * kvq::D * 2 + (size_t)tmax * kvq::D * 2;
                if (!inside(win_off, 2, 0, win_hi) || !inside(kb, kvq::D * 2, 0, win_hi) ||
                    !inside(vb, kvq::D * 2, 0, win_hi))
                    return pc.fail("window bytes outside the cache", unit, tmax, split);
            } else {
                if (split >= page_splits) return pc.fail("page work in a window split", unit, split, wv);
                if (w.g0 < 0 || (w.g1 > w.g0 && w.g1 > 4 * n_pages))
                    return pc.fail("Key group out of range", unit, w.g0, w.g1);
                for (int g = w.g0; g < w.g1; g++) {
                    if (seen_g[g]++) return pc.fail("Key group read twice", unit, g, split);
                    const int p = g >> 2;
                    if (p >= G.max_pages) return pc.fail("page beyond capacity", unit, p, G.max_pages);
                    const size_t off = page_at(p);
                    if (!inside(off, G.page_bytes, pages_lo, pages_hi))
                        return pc.fail("page bytes outside the page region", unit, p, (long)off);
                }
            }
        }
    }
    for (int g = 0; g < 4 * n_pages; g++)
        if (!seen_g[g]) return pc.fail("Key group never read", unit, g, n_pages);
    for (int t = 0; t < n_res; t++)
        if (!seen_t[t]) return pc.fail("window token never read", unit, t, n_res);
    return KVQ_OK;
}

// The dense kernel's grid for `pl` at the counters (n_pages, n_res).
int check_dense(PlanCheck &pc, const kvq_cache *c, const kvq::DecodePlan &pl, int n_pages,
                int n_res, int gps, size_t ws_bytes) {
    const kvq::Geometry &G = c->G;
    constexpr int NW = kvq::kDecodeWaves;
    if (pl.total_splits > kvq::kMaxCombineSplits)
        return pc.fail("more splits than the combine kernel merges", pl.total_splits, 0, 0);
    if (ws_bytes < kvq::decode_workspace_bytes(G, pl.max_splits))
        return pc.fail("workspace smaller than the plan needs", (long)ws_bytes, 0, 0);
    const int win_splits = pl.total_splits - pl.page_splits;
    if (win_splits < 0 || (n_res > 0 && win_splits * 32 * NW < n_res))
        return pc.fail("window splits do not cover the window", win_splits, n_res, 0);
    const int units = G.B * G.Hkv;
    // every workgroup of the grid maps to a (unit, split) of the plan
    const long grid = (long)pl.total_splits * units;
    std::vector<uint8_t> seen((size_t)grid, 0);
    for (long x = 0; x < grid; x++) {
        int unit, split;
        kvq::dense_split_of((int)x, units, pl.page_splits, win_splits, &unit, &split);
        if (unit < 0 || unit >= units || split < 0 || split >= pl.total_splits)
            return pc.fail("workgroup outside the plan", x, unit, split);
        if (seen[(size_t)unit * pl.total_splits + split]++)
            return pc.fail("workgroup mapped twice", x, unit, split);
    }
    std::vector<uint8_t> sg, st;
    const size_t cache_bytes = cache_bytes_of(G);
    for (int u = 0; u < units; u++) {
        int rc = check_unit(pc, G, u, n_pages, n_res, pl.page_splits, win_splits, gps, NW,
                            pl.max_splits, 0, G.res_base, kvq::res_k_off(G, u), cache_bytes,
                            ws_bytes, [&](int p) { return kvq::page_off(G, u, p); }, sg, st);
        if (rc) return rc;
    }
    return KVQ_OK;
}

// The pool kernel's grid for plan `pl` of pool `p` (whose counters and block
// lists are the ones the plan was made from).
int check_pool(PlanCheck &pc, const kvq_pool *p, const kvq::PoolPlan &pl, size_t ws_bytes) {
    const kvq::Geometry &G = p->G;
    if (ws_bytes < kvq::decode_workspace_bytes(G, pl.max_splits))
        return pc.fail("workspace smaller than the plan needs", (long)ws_bytes, 0, 0);
    const uint32_t grid = pl.page_pref[pl.n_seq] + pl.win_pref[pl.n_seq];
    std::vector<std::vector<uint8_t>> seen(G.B);
    for (int b = 0; b < G.B; b++) {
        const int S = (int)(pl.page_pref[b + 1] - pl.page_pref[b]) / G.Hkv;
        const int W = (int)(pl.win_pref[b + 1] - pl.win_pref[b]) / G.Hkv;
        if ((pl.page_pref[b + 1] - pl.page_pref[b]) % G.Hkv || (pl.win_pref[b + 1] - pl.win_pref[b]) % G.Hkv)
            return pc.fail("split counts not a multiple of the KV heads", b, S, W);
        if (S + W > kvq::kMaxCombineSplits) return pc.fail("more splits than the combine kernel merges", b, S, W);
        seen[b].assign((size_t)G.Hkv * (S + W), 0);
    }
    for (uint32_t x = 0; x < grid; x++) {
        int b, h, split, S;
        kvq::pool_split_of(pl, G.Hkv, x, &b, &h, &split, &S);
        const int W = (int)(pl.win_pref[b + 1] - pl.win_pref[b]) / G.Hkv;
        if (b < 0 || b >= G.B || h < 0 || h >= G.Hkv || split < 0 || split >= S + W)
            return pc.fail("workgroup outside the plan", x, b, split);
        if (seen[b][(size_t)h * (S + W) + split]++) return pc.fail("workgroup mapped twice", x, b, split);
    }
    std::vector<uint8_t> sg, st;
    for (int b = 0; b < G.B; b++) {
        const int S = (int)(pl.page_pref[b + 1] - pl.page_pref[b]) / G.Hkv;
        const int W = (int)(pl.win_pref[b + 1] - pl.win_pref[b]) / G.Hkv;
        for (size_t i = 0; i < seen[b].size(); i++)
            if (!seen[b][i]) return pc.fail("split without a workgroup", b, (long)i, 0);
        if (!p->live[b]) {
            if (S || W) return pc.fail("work for a released sequence", b, S, W);
            continue;
        }
        const int np = pl.n_pages[b], nr = pl.n_res[b];
        if (np > (int)p->blocks[b].size()) return pc.fail("pages beyond the block list", b, np, 0);
        for (int h = 0; h < G.Hkv; h++) {
            const int u = b * G.Hkv + h;
            auto page_at = [&](int pg) {
                const int32_t blk = pg < (int)p->blocks[b].size() ? p->blocks[b][pg] : -1;
                return blk < 0 || blk >= p->n_blocks ? ~(size_t)0
                                                     : ((size_t)blk * G.Hkv + h) * G.page_bytes;
            };
            int rc = check_unit(pc, G, u, np, nr, S, W, pl.gps, 1, pl.max_splits, 0, G.res_base,
                                kvq::res_k_off(G, u), p->table_off, ws_bytes, page_at, sg, st);
            if (rc) return rc;
        }
    }
    return KVQ_OK;
}

// ---------------------------------------------------------------- pool ----
constexpr int kPoolMaxPages = 65535;  // page counts travel as 16-bit values
constexpr int kPoolMaxKvHeads = 63;   // window workgroup prefix sums fit 16 bits

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_pool_config(const kvq_config *c, int32_t n_blocks) {
    int rc = check_config(c);
    if (rc) return rc;
    if (c->batch > kvq::kPoolMaxSeqs || c->max_pages > kPoolMaxPages ||
        c->num_kv_heads > kPoolMaxKvHeads || n_blocks < 1)
        return KVQ_EINVAL;
    return KVQ_OK;
}

// Geometry of a pool plus the byte offsets of its windows and table.
kvq::Geometry pool_geometry(const kvq_config *c, int32_t n_blocks, size_t *table_off,
                            size_t *total) {
    kvq::Geometry G = geometry_of(c);
    const size_t blocks = (size_t)n_blocks * G.Hkv * G.page_bytes;
    G.res_base = align256(blocks);
    const size_t win = (size_t)G.B * G.Hkv * 2 * kvq::R * kvq::D * 2;
    *table_off = align256(G.res_base + win);
    *total = *table_off + (size_t)G.B * G.max_pages * sizeof(int32_t);
    return G;
}

int32_t *pool_table(kvq_pool *p) { return reinterpret_cast<int32_t *>(p->mem + p->table_off); }

// Split plan of one decode launch over the live sequences (slot_of[b] >= 0:
// the fused append's window slot of sequence b).
kvq::PoolPlan pool_plan(const kvq_pool *p, const int *slot_of, int slots = 0) {
    const kvq::Geometry &G = p->G;
    kvq::PoolPlan pl{};
    pl.n_seq = G.B;
    pl.max_splits = max_splits_of(G);
    int64_t unit_groups = 0;
    int units_with_pages = 0, max_groups = 0;
    for (int b = 0; b < G.B; b++) {
        if (!p->live[b]) continue;
        unit_groups += (int64_t)4 * p->n_pages[b] * G.Hkv;
        units_with_pages += p->n_pages[b] > 0 ? G.Hkv : 0;
        max_groups = std::max(max_groups, 4 * p->n_pages[b]);
    }
    // One round of resident waves of page splits (the window splits follow
    // as they drain), equal groups per split across all sequences; several
    // rounds of about kRoundGroups groups when the units alone fill more than
    // a round.
    int gps = 1;
    if (units_with_pages > 0) {
        const int target = slots > 0 ? slots : kvq::pool_decode_slots(G);
        if (target >= units_with_pages)
            gps = (int)std::max<int64_t>(1, (unit_groups + target - 1) / target);
        else
            gps = kRoundGroups;
        gps = std::max(gps, (max_groups + kMaxSplits - 1) / kMaxSplits);
    }
    pl.gps = gps;
    pl.page_pref[0] = 0;
    pl.win_pref[0] = 0;
    for (int b = 0; b < G.B; b++) {
        const bool on = p->live[b] != 0;
        // a sequence given a new token (slot_of[b] >= 0) is planned with it
        const int nres = on ? p->n_res[b] + (slot_of && slot_of[b] >= 0 ? 1 : 0) : 0;
        const int S = on ? (4 * p->n_pages[b] + gps - 1) / gps : 0;
        const int W = on ? (nres + 31) / 32 : 0;
        pl.page_pref[b + 1] = pl.page_pref[b] + (uint32_t)(G.Hkv * S);
        pl.win_pref[b + 1] = (uint16_t)(pl.win_pref[b] + G.Hkv * W);
        pl.n_pages[b] = (uint16_t)(on ? p->n_pages[b] : 0);
        pl.n_res[b] = (uint8_t)nres;
        pl.slot[b] = (uint8_t)(on && slot_of && slot_of[b] >= 0 ? slot_of[b] : kvq::kPoolNoSlot);
    }
    for (int b = G.B; b < kvq::kPoolMaxSeqs; b++) {
        pl.page_pref[b + 1] = pl.page_pref[b];
        pl.win_pref[b + 1] = pl.win_pref[b];
    }
    pl.page_wgs = (int)pl.page_pref[G.B];
    return pl;
}

// Flush every live sequence whose window is full into a new block (checks
// first; nothing changes on error).  *n receives the number of flushes.
int pool_flush_full(kvq_pool *p, hipStream_t st, int32_t *n) {
    const kvq::Geometry &G = p->G;
    int need = 0;
    for (int b = 0; b < G.B; b++) {
        if (!p->live[b] || p->n_res[b] != kvq::R) continue;
        if (p->n_pages[b] >= G.max_pages) return KVQ_ECAPACITY;
        need++;
    }
    if (need > (int)p->free_list.size()) return KVQ_ECAPACITY;
    *n = need;
    if (need == 0) return KVQ_OK;
    kvq::PoolPages pp{};
    pp.n = 0;
    for (int b = 0; b < G.B; b++) {
        if (!p->live[b] || p->n_res[b] != kvq::R) continue;
        const int32_t blk = p->free_list[p->free_list.size() - 1 - pp.n];
        pp.block[pp.n] = blk;
        pp.tslot[pp.n] = b * G.max_pages + p->n_pages[b];
        pp.src[pp.n] = b;
        pp.n++;
    }
    const uint16_t *kw = reinterpret_cast<const uint16_t *>(p->mem + G.res_base);
    hipError_t e = kvq::launch_pool_pages(G, p->mem, pool_table(p), kw, kw + (size_t)kvq::R * kvq::D,
                                          (size_t)2 * kvq::R * kvq::D,
                                          (size_t)G.Hkv * 2 * kvq::R * kvq::D, pp, p->rel, st);
    if (e != hipSuccess) return KVQ_EHIP;
    for (int e2 = 0; e2 < pp.n; e2++) {
        const int b = pp.src[e2];
        p->free_list.pop_back();
        p->blocks[b].push_back(pp.block[e2]);
        p->n_pages[b] += 1;
        p->n_res[b] = 0;
    }
    return KVQ_OK;
}

}  // namespace

// ------------------------------------------------------------- prefill ----
namespace {
constexpr int64_t kPrefillMaxT = 1 << 20;  // positions of one prefill
hipEvent_t g_prefill_ev_before = nullptr, g_prefill_ev_after = nullptr;
int g_prefill_max_key_splits = 0;  // 0 = automatic

size_t prefill_stats_bytes(int32_t T, int32_t Hq) { return align256((size_t)Hq * T * 4); }
size_t prefill_part_bytes(int32_t T, int32_t Hkv) {
    return align256((size_t)Hkv * kvq::kColsumChunks * T * 4);
}
size_t prefill_vt_bytes(int32_t T, int32_t Hkv) {
    const size_t T32 = ((size_t)T + 31) / 32 * 32;
    return align256((size_t)Hkv * kvq::D * T32 * 2);
}
// partials of the key-split attention (none when the keys are not split)
size_t prefill_split_bytes(int32_t T, int32_t Hq, int32_t Hkv) {
    int kbc;
    const int s = kvq::prefill_key_splits(T, Hq, Hkv, &kbc);
    return s > 1 ? align256((size_t)Hq * T * s * 2 * 4) + align256((size_t)Hq * T * s * kvq::D * 4)
                 : 0;
}
size_t prefill_ws_bytes(int32_t T, int32_t Hq, int32_t Hkv) {
    return prefill_stats_bytes(T, Hq) + prefill_part_bytes(T, Hkv) + prefill_vt_bytes(T, Hkv) +
           prefill_split_bytes(T, Hq, Hkv);
}
int prefill_shape_ok(int32_t T, int32_t Hq, int32_t Hkv) {
    return T >= 1 && T <= kPrefillMaxT && Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0 &&
           Hq / Hkv <= 16 && (int64_t)Hq * T * kvq::D <= (int64_t)1 << 31;
}
// Runtime debugging switches, read once from the environment:
//   KVQ_CHECK=1  every decode call first walks its launch with the extent
//                check (check_dense / check_pool) and is refused with
//                KVQ_EINVAL, before anything is launched, on a violation;
//   KVQ_TRACE=1  one line per call on stderr (entry point, shape, counters,
//                split plan).
struct DebugFlags {
    bool check, trace;
};
bool env_on(const char *name) {
    const char *v = std::getenv(name);
    return v && *v && *v != '0';
}
const DebugFlags &debug_flags() {
    static const DebugFlags f{env_on("KVQ_CHECK"), env_on("KVQ_TRACE")};
    return f;
}
int debug_dense(const char *who, const kvq_cache *c, const kvq::DecodePlan &pl, int np, int nr,
                int gps, size_t ws_bytes) {
    const DebugFlags &f = debug_flags();
    if (f.trace)
        std::fprintf(stderr, "[kvq] %s: B=%d Hq=%d Hkv=%d k=%d pages=%d window=%d splits=%d+%d "
                     "groups/wave=%d\n", who, c->G.B, c->G.Hq, c->G.Hkv, c->G.k, np, nr,
                     pl.page_splits, pl.total_splits - pl.page_splits, gps);
    if (!f.check) return KVQ_OK;
    char msg[256];
    PlanCheck pc{msg, sizeof msg};
    const int rc = check_dense(pc, c, pl, np, nr, gps, ws_bytes);
    if (rc) std::fprintf(stderr, "[kvq] %s: launch refused (KVQ_CHECK): %s\n", who, msg);
    return rc;
}
int debug_pool(const char *who, const kvq_pool *p, const kvq::PoolPlan &pl, size_t ws_bytes) {
    const DebugFlags &f = debug_flags();
    if (f.trace)
        std::fprintf(stderr, "[kvq] %s: slots=%d Hq=%d Hkv=%d k=%d workgroups=%u+%u groups/split=%d\n",
                     who, p->G.B, p->G.Hq, p->G.Hkv, p->G.k, pl.page_pref[pl.n_seq],
                     (unsigned)pl.win_pref[pl.n_seq], pl.gps);
    if (!f.check) return KVQ_OK;
    char msg[256];
    PlanCheck pc{msg, sizeof msg};
    const int rc = check_pool(pc, p, pl, ws_bytes);
    if (rc) std::fprintf(stderr, "[kvq] %s: launch refused (KVQ_CHECK): %s\n", who, msg);
    return rc;
}
void debug_trace(const char *who, int a, int b, int c2) {
    if (debug_flags().trace) std::fprintf(stderr, "[kvq] %s: %d %d %d\n", who, a, b, c2);
}

}  // namespace

extern "C" {

int kvq_cache_bytes(const kvq_config *cfg, size_t *bytes) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!bytes) return KVQ_EINVAL;
    *bytes = cache_bytes_of(geometry_of(cfg));
    return KVQ_OK;
}

int kvq_page_bytes(const kvq_config *cfg, size_t *bytes) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!bytes) return KVQ_EINVAL;
    *bytes = kvq::page_layout(cfg->boost_channels).bytes;
    return KVQ_OK;
}

int kvq_cache_create(const kvq_config *cfg, void *dev_mem, size_t bytes, kvq_cache **out) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!out || !dev_mem) return KVQ_EINVAL;
    if (!aligned16(dev_mem)) return KVQ_EALIGN;
    kvq::Geometry G = geometry_of(cfg);
    if (bytes < cache_bytes_of(G)) return KVQ_EINVAL;
    kvq_cache *c = new (std::nothrow) kvq_cache;
    if (!c) return KVQ_EINVAL;
    c->G = G;
    c->mem = static_cast<uint8_t *>(dev_mem);
    c->bytes = bytes;
    c->n_pages = 0;
    c->n_res = 0;
    c->splits_override = 0;
    c->rel = nullptr;
    c->ev_before = nullptr;
    c->ev_after = nullptr;
    *out = c;
    return KVQ_OK;
}

int kvq_cache_destroy(kvq_cache *cache) {
    if (!cache) return KVQ_EINVAL;
    delete cache;
    return KVQ_OK;
}

int kvq_quantize_page(kvq_cache *c, const void *k, const void *v, int32_t n_pages,
                      void *stream) {
    if (!c || n_pages < 0) return KVQ_EINVAL;
    if (n_pages == 0) return KVQ_OK;
    if (!k || !v) return KVQ_EINVAL;
    if (!aligned16(k) || !aligned16(v)) return KVQ_EALIGN;
    if (c->n_res != 0) return KVQ_ESTATE;
    if ((int64_t)c->n_pages + n_pages > c->G.max_pages) return KVQ_ECAPACITY;
    hipError_t e = kvq::launch_quantize_pages(
        c->G, c->mem, static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
        (size_t)n_pages * kvq::P * kvq::D, c->n_pages, n_pages, c->rel,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return KVQ_EHIP;
    c->n_pages += n_pages;
    debug_trace("kvq_quantize_page: new pages, pages, window", n_pages, c->n_pages, c->n_res);
    return KVQ_OK;
}

int kvq_append_token(kvq_cache *c, const void *k, const void *v, void *stream,
                     int32_t *flushed) {
    if (!c || !k || !v) return KVQ_EINVAL;
    if (!aligned16(k) || !aligned16(v)) return KVQ_EALIGN;
    bool flush = c->n_res == kvq::R;
    if (flush && c->n_pages >= c->G.max_pages) return KVQ_ECAPACITY;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (flush) {
        hipError_t e = kvq::launch_flush_window(c->G, c->mem, c->n_pages, c->rel, st);
        if (e != hipSuccess) return KVQ_EHIP;
        c->n_pages += 1;
        c->n_res = 0;
    }
    hipError_t e = kvq::launch_append(c->G, c->mem, static_cast<const uint16_t *>(k),
                                      static_cast<const uint16_t *>(v), c->n_res, st);
    if (e != hipSuccess) return KVQ_EHIP;
    c->n_res += 1;
    if (flushed) *flushed = flush ? 1 : 0;
    debug_trace("kvq_append_token: flushed, pages, window", flush ? 1 : 0, c->n_pages, c->n_res);
    return KVQ_OK;
}

int kvq_decode_workspace_bytes(const kvq_cache *c, size_t *bytes) {
    if (!c || !bytes) return KVQ_EINVAL;
    *bytes = kvq::decode_workspace_bytes(c->G, max_splits_of(c->G));
    return KVQ_OK;
}

int kvq_decode_attention(kvq_cache *c, const void *q, float *out, void *workspace,
                         size_t ws_bytes, void *stream) {
    if (!c || !q || !out || !workspace) return KVQ_EINVAL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_EALIGN;
    if (ws_bytes < kvq::decode_workspace_bytes(c->G, max_splits_of(c->G)))
        return KVQ_EWORKSPACE;
    if (c->n_pages == 0 && c->n_res == 0) return KVQ_EEMPTY;
    kvq::DecodePlan pl = plan_of(c);
    if (debug_dense("kvq_decode_attention", c, pl, c->n_pages, c->n_res, pl.groups_per_split, ws_bytes))
        return KVQ_EINVAL;
    return hip_status(kvq::launch_decode(c->G, c->mem, static_cast<const uint16_t *>(q), out,
                                         workspace, pl, nullptr, nullptr, -1, c->ev_before,
                                         c->ev_after, static_cast<hipStream_t>(stream)));
}

int kvq_decode_attention_noalloc(kvq_cache *c, const void *q, float *out, void *stream) {
    if (!c || !q || !out) return KVQ_EINVAL;
    if (!aligned16(q) || !aligned16(out)) return KVQ_EALIGN;
    if (c->n_pages == 0 && c->n_res == 0) return KVQ_EEMPTY;
    kvq::DecodePlan pl = plan_of(c);
    pl.max_splits = pl.total_splits;  // partial stride: only the splits this launch writes
    if (kvq::decode_workspace_bytes(c->G, pl.max_splits) > kvq::kStaticScratchBytes)
        return KVQ_EWORKSPACE;
    if (debug_dense("kvq_decode_attention_noalloc", c, pl, c->n_pages, c->n_res,
                    pl.groups_per_split, kvq::kStaticScratchBytes))
        return KVQ_EINVAL;
    void *ws = nullptr;
    if (kvq::static_scratch(&ws) != hipSuccess) return KVQ_EHIP;
    return hip_status(kvq::launch_decode(c->G, c->mem, static_cast<const uint16_t *>(q), out, ws,
                                         pl, nullptr, nullptr, -1, c->ev_before, c->ev_after,
                                         static_cast<hipStream_t>(stream)));
}

int kvq_append_decode(kvq_cache *c, const void *k, const void *v, const void *q, float *out,
                      void *workspace, size_t ws_bytes, void *stream, int32_t *flushed) {
    if (!c || !k || !v || !q || !out || !workspace) return KVQ_EINVAL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) ||
        !aligned16(workspace))
        return KVQ_EALIGN;
    if (ws_bytes < kvq::decode_workspace_bytes(c->G, max_splits_of(c->G)))
        return KVQ_EWORKSPACE;
    bool flush = c->n_res == kvq::R;
    if (flush && c->n_pages >= c->G.max_pages) return KVQ_ECAPACITY;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the plan and the kernel see the window (flushed first when full) with
    // the new token in it; the counters move only once the launches that
    // flush and write the token succeeded
    kvq_cache next = *c;
    if (flush) {
        next.n_pages += 1;
        next.n_res = 0;
    }
    const int slot = next.n_res;
    kvq::DecodePlan pl = plan_of(&next, slot + 1);
    if (debug_dense("kvq_append_decode", &next, pl, next.n_pages, slot + 1, pl.groups_per_split,
                    ws_bytes))
        return KVQ_EINVAL;
    if (flush) {
        hipError_t e = kvq::launch_flush_window(c->G, c->mem, c->n_pages, c->rel, st);
        if (e != hipSuccess) return KVQ_EHIP;
        c->n_pages += 1;
        c->n_res = 0;
    }
    hipError_t e = kvq::launch_decode(c->G, c->mem, static_cast<const uint16_t *>(q), out,
                                      workspace, pl, static_cast<const uint16_t *>(k),
                                      static_cast<const uint16_t *>(v), slot, c->ev_before,
                                      c->ev_after, st);
    if (e != hipSuccess) return KVQ_EHIP;
    c->n_res = slot + 1;
    if (flushed) *flushed = flush ? 1 : 0;
    return KVQ_OK;
}

int kvq_device_state_init(kvq_cache *c, int32_t *dev_state, void *stream) {
    if (!c || !dev_state) return KVQ_EINVAL;
    if (!aligned16(dev_state)) return KVQ_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // a replayed step starts with room in its window: a full one is flushed
    // here, as the next step would start by doing (the host counters follow)
    if (c->n_res == kvq::R && c->n_pages < c->G.max_pages) {
        const hipError_t e = kvq::launch_flush_window(c->G, c->mem, c->n_pages, c->rel, st);
        if (e != hipSuccess) return KVQ_EHIP;
        c->n_pages += 1;
        c->n_res = 0;
    }
    debug_trace("kvq_device_state_init: pages, window, -", c->n_pages, c->n_res, 0);
    return hip_status(kvq::launch_state_init(dev_state, c->n_pages, c->n_res, st));
}

int kvq_append_decode_device(kvq_cache *c, const void *k, const void *v, const void *q,
                             float *out, void *workspace, size_t ws_bytes, int32_t *dev_state,
                             void *stream) {
    if (!c || !k || !v || !q || !out || !workspace || !dev_state) return KVQ_EINVAL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) ||
        !aligned16(workspace) || !aligned16(dev_state))
        return KVQ_EALIGN;
    if (ws_bytes < kvq::decode_workspace_bytes(c->G, max_splits_of(c->G)))
        return KVQ_EWORKSPACE;
    kvq::DecodePlan pl = device_step_plan(c);
    pl.dstate = dev_state;
    pl.rel = c->rel;
    {
        // the step the host counters describe (the device counters may have
        // moved on; KVQ_CHECK walks the state they would have next)
        const bool full = c->n_res == kvq::R && c->n_pages < c->G.max_pages;
        const int np = full ? c->n_pages + 1 : c->n_pages;
        const int nr = full ? 1 : std::min(c->n_res + 1, (int)kvq::R);
        if (debug_dense("kvq_append_decode_device", c, pl, np, nr, device_step_gps(pl, np), ws_bytes))
            return KVQ_EINVAL;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(kvq::launch_decode(c->G, c->mem, static_cast<const uint16_t *>(q), out,
                                         workspace, pl, static_cast<const uint16_t *>(k),
                                         static_cast<const uint16_t *>(v), 0, c->ev_before,
                                         c->ev_after, st));
}

int kvq_check_decode_plan(const kvq_cache *c, int32_t mode, int32_t slots, size_t ws_bytes,
                          char *msg, size_t msg_len) {
    if (!c || mode < 0 || mode > 2 || slots < 0) return KVQ_EINVAL;
    PlanCheck pc{msg, msg_len};
    if (msg && msg_len) msg[0] = 0;
    if (mode == 0) {
        if (c->n_pages == 0 && c->n_res == 0) return KVQ_OK;  // the call is refused before any launch
        const kvq::DecodePlan pl = plan_of(c, c->n_res, slots);
        return check_dense(pc, c, pl, c->n_pages, c->n_res, pl.groups_per_split, ws_bytes);
    }
    if (mode == 1) {  // kvq_append_decode: flush a full window first, then one more token
        kvq_cache t = *c;
        if (t.n_res == kvq::R) {
            if (t.n_pages >= t.G.max_pages) return KVQ_OK;  // refused before any launch
            t.n_pages += 1;
            t.n_res = 0;
        }
        const kvq::DecodePlan pl = plan_of(&t, t.n_res + 1, slots);
        return check_dense(pc, &t, pl, t.n_pages, t.n_res + 1, pl.groups_per_split, ws_bytes);
    }
    // mode 2: the graph-replayable step captured now, replayed until the
    // cache is full: page split count fixed, groups per wave from the device
    // counters of each replay
    const kvq::DecodePlan pl = device_step_plan(c, slots);
    const int lo = std::max(c->n_pages, 0), hi = c->G.max_pages;
    const int pages[] = {lo, std::min(lo + 1, hi), (lo + hi) / 2, std::max(hi - 1, lo), hi};
    const int wins[] = {1, 2, 31, 32, 33, 64, 97, 127, 128};
    for (int np : pages)
        for (int nr : wins) {
            kvq::DecodePlan q = pl;
            q.n_pages = np;
            q.n_res = nr;
            const int rc = check_dense(pc, c, q, np, nr, device_step_gps(pl, np), ws_bytes);
            if (rc) return rc;
        }
    return KVQ_OK;
}

int kvq_pool_check_decode_plan(const kvq_pool *p, int32_t mode, int32_t slots, size_t ws_bytes,
                               char *msg, size_t msg_len) {
    if (!p || mode < 0 || mode > 1 || slots < 0) return KVQ_EINVAL;
    PlanCheck pc{msg, msg_len};
    if (msg && msg_len) msg[0] = 0;
    if (mode == 0) return check_pool(pc, p, pool_plan(p, nullptr, slots), ws_bytes);
    // kvq_pool_append_decode: full windows flushed into the next free blocks
    // first, then one more token per live sequence
    kvq_pool t = *p;
    for (int b = 0; b < t.G.B; b++) {
        if (!t.live[b] || t.n_res[b] != kvq::R) continue;
        if (t.free_list.empty() || t.n_pages[b] >= t.G.max_pages) return KVQ_OK;  // refused first
        t.blocks[b].push_back(t.free_list.back());
        t.free_list.pop_back();
        t.n_pages[b] += 1;
        t.n_res[b] = 0;
    }
    int slot_of[kvq::kPoolMaxSeqs];
    for (int b = 0; b < t.G.B; b++) slot_of[b] = t.live[b] ? t.n_res[b] : -1;
    return check_pool(pc, &t, pool_plan(&t, slot_of, slots), ws_bytes);
}

int kvq_set_decode_splits(kvq_cache *c, int32_t splits) {
    if (!c || splits < 0) return KVQ_EINVAL;
    c->splits_override = splits;
    return KVQ_OK;
}

int kvq_get_decode_splits(const kvq_cache *c, int32_t *splits) {
    if (!c || !splits) return KVQ_EINVAL;
    *splits = plan_of(c).page_splits;
    return KVQ_OK;
}

int kvq_get_state(const kvq_cache *c, int32_t *n_pages, int32_t *n_res) {
    if (!c) return KVQ_EINVAL;
    if (n_pages) *n_pages = c->n_pages;
    if (n_res) *n_res = c->n_res;
    return KVQ_OK;
}

int kvq_set_state(kvq_cache *c, int32_t n_pages, int32_t n_res) {
    if (!c || n_pages < 0 || n_pages > c->G.max_pages || n_res < 0 || n_res > kvq::R)
        return KVQ_EINVAL;
    c->n_pages = n_pages;
    c->n_res = n_res;
    return KVQ_OK;
}

int kvq_page_offset(const kvq_cache *c, int32_t b, int32_t h, int32_t page, size_t *off) {
    if (!c || !off || b < 0 || b >= c->G.B || h < 0 || h >= c->G.Hkv || page < 0 ||
        page >= c->G.max_pages)
        return KVQ_EINVAL;
    *off = kvq::page_off(c->G, b * c->G.Hkv + h, page);
    return KVQ_OK;
}

int kvq_residual_offset(const kvq_cache *c, int32_t b, int32_t h, size_t *k_off,
                        size_t *v_off) {
    if (!c || b < 0 || b >= c->G.B || h < 0 || h >= c->G.Hkv) return KVQ_EINVAL;
    int u = b * c->G.Hkv + h;
    if (k_off) *k_off = kvq::res_k_off(c->G, u);
    if (v_off) *v_off = kvq::res_v_off(c->G, u);
    return KVQ_OK;
}

int kvq_quantize_groups(int32_t dtype, int32_t L, const void *x, int32_t n_groups,
                        int32_t group_len, void *s, void *z, void *codes, void *stream) {
    if (dtype != KVQ_F16 && dtype != KVQ_BF16) return KVQ_EINVAL;
    if (L != 3 && L != 15) return KVQ_EINVAL;
    if (n_groups < 0 || group_len < 1 || group_len > 256) return KVQ_EINVAL;
    if (n_groups == 0) return KVQ_OK;
    if (!x || !s || !z || !codes) return KVQ_EINVAL;
    return hip_status(kvq::launch_quantize_groups(
        dtype, L, static_cast<const uint16_t *>(x), n_groups, group_len,
        static_cast<uint16_t *>(s), static_cast<uint16_t *>(z), static_cast<uint8_t *>(codes),
        static_cast<hipStream_t>(stream)));
}

int kvq_set_channel_relevance(kvq_cache *c, const float *rel) {
    if (!c) return KVQ_EINVAL;
    if (rel && !aligned16(rel)) return KVQ_EALIGN;
    c->rel = rel;
    return KVQ_OK;
}


int kvq_prefill_workspace_bytes(int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                size_t *bytes) {
    if (!bytes || !prefill_shape_ok(T, num_q_heads, num_kv_heads)) return KVQ_EINVAL;
    *bytes = prefill_ws_bytes(T, num_q_heads, num_kv_heads);
    return KVQ_OK;
}

int kvq_prefill_select(int32_t dtype, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                       float softmax_scale, const void *q, const void *k, const void *v,
                       int32_t heavy, int32_t recent, float *out, float *score, int32_t *keep,
                       void *k_sel, void *v_sel, void *workspace, size_t ws_bytes, void *stream,
                       int32_t *n_keep) {
    if (dtype != KVQ_F16 && dtype != KVQ_BF16) return KVQ_EINVAL;
    if (!prefill_shape_ok(T, num_q_heads, num_kv_heads) || heavy < 0 || recent < 0)
        return KVQ_EINVAL;
    if (!q || !k || !v || !out || !score || !workspace || !n_keep) return KVQ_EINVAL;
    if (!k_sel != !v_sel) return KVQ_EINVAL;
    const int32_t rec = std::min(recent, T);
    const int32_t hv = std::min(heavy, T - rec);
    const int32_t nk = hv + rec;
    if (nk > 0 && !keep) return KVQ_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(score) ||
        !aligned16(workspace) || (keep && !aligned16(keep)) || (k_sel && !aligned16(k_sel)) ||
        (v_sel && !aligned16(v_sel)))
        return KVQ_EALIGN;
    if (ws_bytes < prefill_ws_bytes(T, num_q_heads, num_kv_heads)) return KVQ_EWORKSPACE;
    kvq::PrefillArgs a{};
    a.T = T;
    a.T32 = (T + 31) / 32 * 32;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.heavy = heavy;
    a.recent = recent;
    a.n_keep = nk;
    a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)kvq::D);
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    a.lse = reinterpret_cast<float *>(ws);
    a.part = reinterpret_cast<float *>(ws + prefill_stats_bytes(T, num_q_heads));
    a.vt = reinterpret_cast<uint16_t *>(ws + prefill_stats_bytes(T, num_q_heads) +
                                        prefill_part_bytes(T, num_kv_heads));
    a.nsplit = kvq::prefill_key_splits(T, num_q_heads, num_kv_heads, &a.kbc,
                                       g_prefill_max_key_splits);
    {
        uint8_t *sp = ws + prefill_stats_bytes(T, num_q_heads) + prefill_part_bytes(T, num_kv_heads) +
                      prefill_vt_bytes(T, num_kv_heads);
        a.pml = a.nsplit > 1 ? reinterpret_cast<float *>(sp) : nullptr;
        a.pacc = a.nsplit > 1
                     ? reinterpret_cast<float *>(sp + align256((size_t)num_q_heads * T * a.nsplit * 2 * 4))
                     : nullptr;
    }
    a.out = out;
    a.score = score;
    a.keep = keep;
    a.k_sel = static_cast<uint16_t *>(k_sel);
    a.v_sel = static_cast<uint16_t *>(v_sel);
    a.ev_before = g_prefill_ev_before;
    a.ev_after = g_prefill_ev_after;
    *n_keep = nk;
    debug_trace("kvq_prefill_select: tokens, key chunks, kept", T, a.nsplit, nk);
    return hip_status(kvq::launch_prefill(dtype, a, static_cast<hipStream_t>(stream)));
}

int kvq_prefill_set_max_key_splits(int32_t n) {
    if (n < 0 || n > kvq::kPrefillMaxKeySplits) return KVQ_EINVAL;
    g_prefill_max_key_splits = n;
    return KVQ_OK;
}

int kvq_prefill_set_kernel_events(void *before, void *after) {
    if ((before == nullptr) != (after == nullptr)) return KVQ_EINVAL;
    g_prefill_ev_before = static_cast<hipEvent_t>(before);
    g_prefill_ev_after = static_cast<hipEvent_t>(after);
    return KVQ_OK;
}

int kvq_query_relevance(int32_t dtype, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                        const void *q, float *rel, void *stream) {
    if (dtype != KVQ_F16 && dtype != KVQ_BF16) return KVQ_EINVAL;
    if (batch < 0 || num_kv_heads < 1 || num_q_heads < num_kv_heads ||
        num_q_heads % num_kv_heads || (int64_t)batch * num_kv_heads * kvq::D > (1 << 30))
        return KVQ_EINVAL;
    if (batch == 0) return KVQ_OK;
    if (!q || !rel) return KVQ_EINVAL;
    if (!aligned16(q) || !aligned16(rel)) return KVQ_EALIGN;
    return hip_status(kvq::launch_query_relevance(dtype, static_cast<const uint16_t *>(q), rel,
                                                  batch, num_q_heads, num_kv_heads,
                                                  static_cast<hipStream_t>(stream)));
}

int kvq_set_kernel_events(kvq_cache *c, void *before, void *after) {
    if (!c) return KVQ_EINVAL;
    if ((before == nullptr) != (after == nullptr)) return KVQ_EINVAL;
    c->ev_before = static_cast<hipEvent_t>(before);
    c->ev_after = static_cast<hipEvent_t>(after);
    return KVQ_OK;
}

int kvq_pool_bytes(const kvq_config *cfg, int32_t n_blocks, size_t *bytes) {
    int rc = check_pool_config(cfg, n_blocks);
    if (rc) return rc;
    if (!bytes) return KVQ_EINVAL;
    size_t table_off, total;
    pool_geometry(cfg, n_blocks, &table_off, &total);
    *bytes = total;
    return KVQ_OK;
}

int kvq_pool_create(const kvq_config *cfg, int32_t n_blocks, void *dev_mem, size_t bytes,
                    kvq_pool **out) {
    int rc = check_pool_config(cfg, n_blocks);
    if (rc) return rc;
    if (!out || !dev_mem) return KVQ_EINVAL;
    if (!aligned16(dev_mem)) return KVQ_EALIGN;
    size_t table_off, total;
    kvq::Geometry G = pool_geometry(cfg, n_blocks, &table_off, &total);
    if (bytes < total) return KVQ_EINVAL;
    kvq_pool *p = new (std::nothrow) kvq_pool;
    if (!p) return KVQ_EINVAL;
    try {
        p->G = G;
        p->mem = static_cast<uint8_t *>(dev_mem);
        p->bytes = bytes;
        p->table_off = table_off;
        p->n_blocks = n_blocks;
        p->live.assign(G.B, 0);
        p->n_pages.assign(G.B, 0);
        p->n_res.assign(G.B, 0);
        p->blocks.assign(G.B, std::vector<int32_t>());
        p->free_list.resize(n_blocks);
        for (int32_t i = 0; i < n_blocks; i++) p->free_list[i] = n_blocks - 1 - i;
        p->rel = nullptr;
        p->ev_before = nullptr;
        p->ev_after = nullptr;
    } catch (...) {
        delete p;
        return KVQ_EINVAL;
    }
    *out = p;
    return KVQ_OK;
}

int kvq_pool_destroy(kvq_pool *pool) {
    if (!pool) return KVQ_EINVAL;
    delete pool;
    return KVQ_OK;
}

int kvq_pool_prefill(kvq_pool *p, int32_t seq, const void *k, const void *v, int32_t n_tokens,
                     void *stream) {
    if (!p || seq < 0 || seq >= p->G.B || n_tokens < 0) return KVQ_EINVAL;
    if (n_tokens > 0 && (!k || !v)) return KVQ_EINVAL;
    if (n_tokens > 0 && (!aligned16(k) || !aligned16(v))) return KVQ_EALIGN;
    if (p->live[seq]) return KVQ_ESTATE;
    const kvq::Geometry &G = p->G;
    const int n_full = n_tokens / kvq::P, tail = n_tokens % kvq::P;
    if (n_full > G.max_pages || n_full > (int)p->free_list.size()) return KVQ_ECAPACITY;
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::vector<int32_t> got;
    try {
        got.assign(p->free_list.end() - n_full, p->free_list.end());
    } catch (...) {
        return KVQ_EINVAL;
    }
    std::reverse(got.begin(), got.end());  // handed out from the back of the list
    const uint16_t *ks = static_cast<const uint16_t *>(k), *vs = static_cast<const uint16_t *>(v);
    for (int c0 = 0; c0 < n_full; c0 += kvq::kPoolMaxSeqs) {
        kvq::PoolPages pp{};
        pp.n = std::min(kvq::kPoolMaxSeqs, n_full - c0);
        for (int e = 0; e < pp.n; e++) {
            pp.block[e] = got[c0 + e];
            pp.tslot[e] = seq * G.max_pages + c0 + e;
            pp.src[e] = c0 + e;
        }
        hipError_t e = kvq::launch_pool_pages(G, p->mem, pool_table(p), ks, vs,
                                              (size_t)n_tokens * kvq::D,
                                              (size_t)kvq::P * kvq::D, pp, p->rel, st);
        if (e != hipSuccess) return KVQ_EHIP;
    }
    hipError_t e = kvq::launch_pool_window_fill(G, p->mem, ks, vs, seq, n_tokens,
                                                n_full * kvq::P, tail, st);
    if (e != hipSuccess) return KVQ_EHIP;
    p->free_list.resize(p->free_list.size() - n_full);
    p->blocks[seq] = got;
    p->n_pages[seq] = n_full;
    p->n_res[seq] = tail;
    p->live[seq] = 1;
    return KVQ_OK;
}

int kvq_pool_append(kvq_pool *p, const void *k, const void *v, void *stream,
                    int32_t *n_flushed) {
    if (!p || !k || !v) return KVQ_EINVAL;
    if (!aligned16(k) || !aligned16(v)) return KVQ_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t nf = 0;
    int rc = pool_flush_full(p, st, &nf);
    if (rc) return rc;
    kvq::PoolSlots ps{};
    for (int b = 0; b < kvq::kPoolMaxSeqs; b++)
        ps.slot[b] = (uint8_t)(b < p->G.B && p->live[b] ? p->n_res[b] : kvq::kPoolNoSlot);
    hipError_t e = kvq::launch_pool_append(p->G, p->mem, static_cast<const uint16_t *>(k),
                                           static_cast<const uint16_t *>(v), ps, st);
    if (e != hipSuccess) return KVQ_EHIP;
    for (int b = 0; b < p->G.B; b++)
        if (p->live[b]) p->n_res[b] += 1;
    if (n_flushed) *n_flushed = nf;
    return KVQ_OK;
}

int kvq_pool_decode_workspace_bytes(const kvq_pool *p, size_t *bytes) {
    if (!p || !bytes) return KVQ_EINVAL;
    *bytes = kvq::decode_workspace_bytes(p->G, max_splits_of(p->G));
    return KVQ_OK;
}

int kvq_pool_decode_attention(kvq_pool *p, const void *q, float *out, void *workspace,
                              size_t ws_bytes, void *stream) {
    if (!p || !q || !out || !workspace) return KVQ_EINVAL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_EALIGN;
    if (ws_bytes < kvq::decode_workspace_bytes(p->G, max_splits_of(p->G)))
        return KVQ_EWORKSPACE;
    const kvq::PoolPlan pl = pool_plan(p, nullptr);
    if (debug_pool("kvq_pool_decode_attention", p, pl, ws_bytes)) return KVQ_EINVAL;
    return hip_status(kvq::launch_pool_decode(p->G, p->mem, pool_table(p),
                                              static_cast<const uint16_t *>(q), out, workspace,
                                              pl, nullptr, nullptr, p->ev_before, p->ev_after,
                                              static_cast<hipStream_t>(stream)));
}

int kvq_pool_append_decode(kvq_pool *p, const void *k, const void *v, const void *q, float *out,
                           void *workspace, size_t ws_bytes, void *stream, int32_t *n_flushed) {
    if (!p || !k || !v || !q || !out || !workspace) return KVQ_EINVAL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) ||
        !aligned16(workspace))
        return KVQ_EALIGN;
    if (ws_bytes < kvq::decode_workspace_bytes(p->G, max_splits_of(p->G)))
        return KVQ_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_flags().check) {  // the launch this call makes, walked before the flushes
        char msg[256];
        if (kvq_pool_check_decode_plan(p, 1, 0, ws_bytes, msg, sizeof msg)) {
            std::fprintf(stderr, "[kvq] kvq_pool_append_decode: launch refused (KVQ_CHECK): %s\n", msg);
            return KVQ_EINVAL;
        }
    }
    int32_t nf = 0;
    int rc = pool_flush_full(p, st, &nf);
    if (rc) return rc;
    // the plan and the kernel see every window with its new token in it
    // (the host counters move only once the launch that writes the tokens
    // succeeded)
    int slot_of[kvq::kPoolMaxSeqs];
    for (int b = 0; b < p->G.B; b++) slot_of[b] = p->live[b] ? p->n_res[b] : -1;
    const kvq::PoolPlan pl = pool_plan(p, slot_of);
    if (debug_flags().trace) debug_pool("kvq_pool_append_decode", p, pl, ws_bytes);
    hipError_t e = kvq::launch_pool_decode(p->G, p->mem, pool_table(p),
                                           static_cast<const uint16_t *>(q), out, workspace, pl,
                                           static_cast<const uint16_t *>(k),
                                           static_cast<const uint16_t *>(v), p->ev_before,
                                           p->ev_after, st);
    if (e != hipSuccess) return KVQ_EHIP;
    for (int b = 0; b < p->G.B; b++)
        if (p->live[b]) p->n_res[b] += 1;
    if (n_flushed) *n_flushed = nf;
    return KVQ_OK;
}

int kvq_pool_release(kvq_pool *p, int32_t seq) {
    if (!p || seq < 0 || seq >= p->G.B) return KVQ_EINVAL;
    if (!p->live[seq]) return KVQ_ESTATE;
    std::vector<int32_t> &bl = p->blocks[seq];
    for (auto it = bl.rbegin(); it != bl.rend(); ++it) p->free_list.push_back(*it);
    bl.clear();
    p->live[seq] = 0;
    p->n_pages[seq] = 0;
    p->n_res[seq] = 0;
    return KVQ_OK;
}

int kvq_pool_get_seq(const kvq_pool *p, int32_t seq, int32_t *live, int32_t *n_pages,
                     int32_t *n_res) {
    if (!p || seq < 0 || seq >= p->G.B) return KVQ_EINVAL;
    if (live) *live = p->live[seq];
    if (n_pages) *n_pages = p->n_pages[seq];
    if (n_res) *n_res = p->n_res[seq];
    return KVQ_OK;
}

int kvq_pool_block_of(const kvq_pool *p, int32_t seq, int32_t page, int32_t *block) {
    if (!p || !block || seq < 0 || seq >= p->G.B || !p->live[seq] || page < 0 ||
        page >= p->n_pages[seq])
        return KVQ_EINVAL;
    *block = p->blocks[seq][page];
    return KVQ_OK;
}

int kvq_pool_free_blocks(const kvq_pool *p, int32_t *n_free) {
    if (!p || !n_free) return KVQ_EINVAL;
    *n_free = (int32_t)p->free_list.size();
    return KVQ_OK;
}

int kvq_pool_page_offset(const kvq_pool *p, int32_t block, int32_t h, size_t *off) {
    if (!p || !off || block < 0 || block >= p->n_blocks || h < 0 || h >= p->G.Hkv)
        return KVQ_EINVAL;
    *off = ((size_t)block * p->G.Hkv + h) * p->G.page_bytes;
    return KVQ_OK;
}

int kvq_pool_window_offset(const kvq_pool *p, int32_t seq, int32_t h, size_t *k_off,
                           size_t *v_off) {
    if (!p || seq < 0 || seq >= p->G.B || h < 0 || h >= p->G.Hkv) return KVQ_EINVAL;
    const int u = seq * p->G.Hkv + h;
    if (k_off) *k_off = kvq::res_k_off(p->G, u);
    if (v_off) *v_off = kvq::res_v_off(p->G, u);
    return KVQ_OK;
}

int kvq_pool_table_offset(const kvq_pool *p, size_t *off) {
    if (!p || !off) return KVQ_EINVAL;
    *off = p->table_off;
    return KVQ_OK;
}

int kvq_pool_set_channel_relevance(kvq_pool *p, const float *rel) {
    if (!p) return KVQ_EINVAL;
    if (rel && !aligned16(rel)) return KVQ_EALIGN;
    p->rel = rel;
    return KVQ_OK;
}

int kvq_pool_set_kernel_events(kvq_pool *p, void *before, void *after) {
    if (!p) return KVQ_EINVAL;
    if ((before == nullptr) != (after == nullptr)) return KVQ_EINVAL;
    p->ev_before = static_cast<hipEvent_t>(before);
    p->ev_after = static_cast<hipEvent_t>(after);
    return KVQ_OK;
}

int kvq_probe_bandwidth(int32_t mode, const void *src, void *dst, size_t bytes, void *stream) {
    if ((mode != 0 && mode != 1) || !src || !dst || bytes == 0 || bytes % 16) return KVQ_EINVAL;
    if (!aligned16(src) || !aligned16(dst)) return KVQ_EALIGN;
    return hip_status(kvq::launch_probe(mode, src, dst, bytes, static_cast<hipStream_t>(stream)));
}

const char *kvq_strerror(int code) {
    switch (code) {
        case KVQ_OK: return "ok";
        case KVQ_EINVAL: return "invalid configuration or argument";
        case KVQ_ECAPACITY: return "page capacity exceeded";
        case KVQ_ESTATE: return "call not allowed in the current cache state";
        case KVQ_EEMPTY: return "attention over an empty cache";
        case KVQ_EWORKSPACE: return "workspace too small";
        case KVQ_EALIGN: return "device pointer not 16-byte aligned";
        case KVQ_EHIP: return "HIP launch failed";
        default: return "unknown error";
    }
}

}  // extern "C"
