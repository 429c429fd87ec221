// kvq_host.cpp -- the C ABI of include/kvq.h: configuration checks, cache
// layout and counters, decode planning and kernel launches.  Never allocates
// or frees device memory and never synchronizes; every check happens before
// any launch so a failed call leaves the cache unchanged.
#include "../../include/kvq.h"

#include <cmath>
#include <cstdlib>
#include <new>

#include "kvq_internal.h"

struct kvq_cache {
    kvq::Geometry G;
    uint8_t *mem;
    size_t bytes;
    int32_t n_pages;
    int32_t n_res;
    int32_t splits_override;  // 0 = automatic
    hipEvent_t ev_before, ev_after;
};

namespace {

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

kvq::DecodePlan plan_of(const kvq_cache *c) {
    kvq::DecodePlan pl{};
    pl.n_pages = c->n_pages;
    pl.n_res = c->n_res;
    pl.max_splits = max_splits_of(c->G);
    if (c->n_pages > 0) {
        int S;
        if (c->splits_override > 0) {
            S = c->splits_override;
        } else {
            // One round of resident single-wave workgroups (occupancy of this
            // kernel instance x compute units), shared with the window
            // splits, with equal groups per split.  When the units alone fill
            // more than a round, splits of about kRoundGroups groups run in
            // several rounds and the hardware's dispatch balances them.
            int units = c->G.B * c->G.Hkv;
            int win = (c->n_res + 31) / 32;
            int per_unit = kvq::decode_slots(c->G) / units - win;
            S = per_unit >= 1 ? per_unit : (4 * c->n_pages + kRoundGroups - 1) / kRoundGroups;
        }
        const int groups = 4 * c->n_pages;
        S = std::max(1, std::min(S, std::min(groups, kMaxSplits)));
        pl.groups_per_split = (groups + S - 1) / S;
        pl.page_splits = (groups + pl.groups_per_split - 1) / pl.groups_per_split;
    }
    pl.total_splits = pl.page_splits + (c->n_res + 31) / 32;
    return pl;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_EHIP; }

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
        (size_t)n_pages * kvq::P * kvq::D, c->n_pages, n_pages,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return KVQ_EHIP;
    c->n_pages += n_pages;
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
        hipError_t e = kvq::launch_flush_window(c->G, c->mem, c->n_pages, st);
        if (e != hipSuccess) return KVQ_EHIP;
        c->n_pages += 1;
        c->n_res = 0;
    }
    hipError_t e = kvq::launch_append(c->G, c->mem, static_cast<const uint16_t *>(k),
                                      static_cast<const uint16_t *>(v), c->n_res, st);
    if (e != hipSuccess) return KVQ_EHIP;
    c->n_res += 1;
    if (flushed) *flushed = flush ? 1 : 0;
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
    return hip_status(kvq::launch_decode(c->G, c->mem, static_cast<const uint16_t *>(q), out,
                                         workspace, pl, nullptr, nullptr, -1, c->ev_before,
                                         c->ev_after, static_cast<hipStream_t>(stream)));
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
    if (flush) {
        hipError_t e = kvq::launch_flush_window(c->G, c->mem, c->n_pages, st);
        if (e != hipSuccess) return KVQ_EHIP;
        c->n_pages += 1;
        c->n_res = 0;
    }
    // the plan and the kernel see the window with the new token in it
    const int slot = c->n_res;
    c->n_res += 1;
    kvq::DecodePlan pl = plan_of(c);
    hipError_t e = kvq::launch_decode(c->G, c->mem, static_cast<const uint16_t *>(q), out,
                                      workspace, pl, static_cast<const uint16_t *>(k),
                                      static_cast<const uint16_t *>(v), slot, c->ev_before,
                                      c->ev_after, st);
    if (e != hipSuccess) return KVQ_EHIP;
    if (flushed) *flushed = flush ? 1 : 0;
    return KVQ_OK;
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

int kvq_set_kernel_events(kvq_cache *c, void *before, void *after) {
    if (!c) return KVQ_EINVAL;
    if ((before == nullptr) != (after == nullptr)) return KVQ_EINVAL;
    c->ev_before = static_cast<hipEvent_t>(before);
    c->ev_after = static_cast<hipEvent_t>(after);
    return KVQ_OK;
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
