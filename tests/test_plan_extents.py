"""Host-side extent check of the decode launches (kvq_check_decode_plan), no
GPU: for every workload shape, query-group size and boost, many cache states
(empty window, full window, one page, full capacity), resident-wave counts
of the split plan and split overrides, and each of the three decode entry
points (attention, fused append + attention, graph-replayable step), every
workgroup and wave of the launch is walked with the kernels' own index
arithmetic: every page, window token and split partial lies inside the
cache and the workspace, every Key group and window token is read exactly
once, and the split count fits the combine kernel.  The check itself is
shown to catch a workspace one byte short.
"""
import dataclasses

import pytest

from bit_mixed_precision_page_amd import inputs as gen

FAKE = 0x7f0000000000  # 16-byte aligned device address, never touched on the host
W = gen.WORKLOADS


@pytest.fixture(scope="module")
def kvq():
    from bit_mixed_precision_page_amd import kvq
    return kvq


def _cases():
    out = []
    for name in ("tiny", "llama3_8b_decode", "qwen3_8b_long", "llama70b_large_batch",
                 "long_prefill_decode"):
        out.append((name, W[name]))
    base = W["llama3_8b_decode"]
    for g in (1, 2, 8, 16):
        out.append((f"g{g}", dataclasses.replace(base, B=3, Hkv=2, Hq=2 * g, ctx=2048)))
    for k in (0, 48, 128):
        out.append((f"k{k}", dataclasses.replace(base, B=2, boost=k, ctx=1024)))
    return out


def _states(max_pages):
    pages = sorted({0, 1, 2, 3, 7, max_pages // 2, max_pages - 1, max_pages})
    return [(p, r) for p in pages for r in (0, 1, 31, 32, 33, 127, 128) if p + r > 0]


@pytest.mark.parametrize("name,w", _cases(), ids=[c[0] for c in _cases()])
def test_decode_plans_stay_inside_their_buffers(kvq, name, w):
    cfg = kvq.config(w.B, w.Hq, w.Hkv, w.boost, w.max_pages, w.dtype)
    n = kvq.kvq_cache_bytes(cfg)
    h = kvq.kvq_cache_create(cfg, FAKE, n)
    try:
        ws = kvq.kvq_decode_workspace_bytes(h)
        states = _states(w.max_pages)
        big = w.B * w.Hkv * w.max_pages > 20000
        slots_list = (3072, 4096) if big else (256, 1024, 3072, 4096, 16384)
        splits_list = (0, 5) if big else (0, 1, 3, 7, 64, 1000)
        checked = 0
        for n_pages, n_res in (states[::3] if big else states):
            kvq.kvq_set_state(h, n_pages, n_res)
            for splits in splits_list:
                kvq.kvq_set_decode_splits(h, splits)
                for slots in slots_list:
                    for mode in (0, 1, 2):
                        if mode == 2 and n_pages == w.max_pages and n_res == 128:
                            continue  # the step would only raise the full-cache flag
                        rc, msg = kvq.kvq_check_decode_plan(h, mode, slots, ws)
                        assert rc == 0, (name, n_pages, n_res, splits, slots, mode, msg)
                        checked += 1
        assert checked > 0
    finally:
        kvq.kvq_cache_destroy(h)


def test_check_catches_a_short_workspace(kvq):
    w = W["llama3_8b_decode"]
    cfg = kvq.config(2, w.Hq, w.Hkv, w.boost, 8, w.dtype)
    h = kvq.kvq_cache_create(cfg, FAKE, kvq.kvq_cache_bytes(cfg))
    try:
        kvq.kvq_set_state(h, 5, 40)
        ws = kvq.kvq_decode_workspace_bytes(h)
        assert kvq.kvq_check_decode_plan(h, 0, 4096, ws)[0] == 0
        rc, msg = kvq.kvq_check_decode_plan(h, 0, 4096, ws - 1)
        assert rc != 0 and "workspace" in msg
        with pytest.raises(kvq.KvqError):
            kvq._check(kvq._L.kvq_check_decode_plan(h, 3, 0, ws, None, 0), "mode")
    finally:
        kvq.kvq_cache_destroy(h)
