"""C-ABI tests that need no GPU: the library loads, exports every declared
symbol, and rejects bad calls with the documented codes before any launch.

Handles below wrap a fake, never-dereferenced device address: every call
checked here returns before launching a kernel.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")
FAKE = 0x7f0000000000  # 16-byte aligned, never touched by host-side checks


@pytest.fixture(scope="module")
def kvq():
    from bit_mixed_precision_page_amd import kvq
    return kvq


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(kvq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    syms = declared_symbols()
    for name in ("kvq_quantize_page", "kvq_append_token", "kvq_decode_attention",
                 "kvq_append_decode"):
        assert name in syms
    assert len(syms) >= 18


def test_library_exports_every_declared_symbol(kvq):
    lib = ctypes.CDLL(kvq.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), f"{name} not exported"
    assert set(declared_symbols()) == set(kvq.EXPORTS)


def _cfg(kvq, **kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, boost_channels=16, max_pages=4,
                dtype=kvq.KVQ_BF16)
    base.update(kw)
    return kvq.config(**base)


def test_sizes_match_the_layout(kvq, ora):
    for k in (0, 16, 32, 128):
        c = _cfg(kvq, boost_channels=k)
        pb = kvq.kvq_page_bytes(c)
        assert pb == ora.page_bytes(k)
        assert kvq.kvq_cache_bytes(c) == 2 * 2 * 4 * pb + 2 * 2 * 2 * 128 * 128 * 2
    assert kvq.kvq_page_bytes(_cfg(kvq, boost_channels=16)) == 12816
    assert kvq.kvq_page_bytes(_cfg(kvq, boost_channels=32)) == 13344


@pytest.mark.parametrize("bad", [
    dict(head_dim=64), dict(page_tokens=64), dict(key_group_tokens=16),
    dict(value_group_channels=64), dict(residual_tokens=64), dict(boost_channels=8),
    dict(boost_channels=144), dict(boost_channels=-16), dict(num_q_heads=6),
    dict(num_q_heads=12, num_kv_heads=4), dict(num_q_heads=64, num_kv_heads=2),
    dict(batch=0), dict(max_pages=0), dict(dtype=2), dict(softmax_scale=float("inf")),
])
def test_bad_configs_are_rejected(kvq, bad):
    c = _cfg(kvq, **bad)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_bytes(c)
    assert e.value.name == "KVQ_EINVAL"


def _handle(kvq, **kw):
    c = _cfg(kvq, **kw)
    return kvq.kvq_cache_create(c, FAKE, kvq.kvq_cache_bytes(c)), c


def test_create_checks(kvq):
    c = _cfg(kvq)
    n = kvq.kvq_cache_bytes(c)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_create(c, FAKE + 8, n)
    assert e.value.name == "KVQ_EALIGN"
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_create(c, FAKE, n - 1)
    assert e.value.name == "KVQ_EINVAL"
    h = kvq.kvq_cache_create(c, FAKE, n)
    assert kvq.kvq_get_state(h) == (0, 0)
    kvq.kvq_cache_destroy(h)


def test_call_errors_leave_state_unchanged(kvq):
    h, c = _handle(kvq)
    ws = kvq.kvq_decode_workspace_bytes(h)
    assert ws > 0
    # empty cache
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention(h, FAKE, FAKE, FAKE, ws, 0)
    assert e.value.name == "KVQ_EEMPTY"
    # capacity
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_quantize_page(h, FAKE, FAKE, 5, 0)
    assert e.value.name == "KVQ_ECAPACITY"
    # alignment
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_quantize_page(h, FAKE + 2, FAKE, 1, 0)
    assert e.value.name == "KVQ_EALIGN"
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append_token(h, FAKE, FAKE + 4, 0)
    assert e.value.name == "KVQ_EALIGN"
    # bulk quantization needs an empty window
    kvq.kvq_set_state(h, 1, 5)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_quantize_page(h, FAKE, FAKE, 1, 0)
    assert e.value.name == "KVQ_ESTATE"
    assert kvq.kvq_get_state(h) == (1, 5)
    # workspace
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention(h, FAKE, FAKE, FAKE, ws - 1, 0)
    assert e.value.name == "KVQ_EWORKSPACE"
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention(h, FAKE + 2, FAKE, FAKE, ws, 0)
    assert e.value.name == "KVQ_EALIGN"
    # a full window with no free page cannot flush
    kvq.kvq_set_state(h, 4, 128)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append_token(h, FAKE, FAKE, 0)
    assert e.value.name == "KVQ_ECAPACITY"
    assert kvq.kvq_get_state(h) == (4, 128)
    # the fused step checks like the two calls it replaces, before any launch
    for args, name in [((FAKE, FAKE, FAKE, FAKE, FAKE, ws), "KVQ_ECAPACITY"),
                       ((FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1), "KVQ_EWORKSPACE"),
                       ((FAKE, FAKE + 2, FAKE, FAKE, FAKE, ws), "KVQ_EALIGN"),
                       ((FAKE, FAKE, FAKE, FAKE + 4, FAKE, ws), "KVQ_EALIGN"),
                       ((FAKE, 0, FAKE, FAKE, FAKE, ws), "KVQ_EINVAL")]:
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_append_decode(h, *args, 0)
        assert e.value.name == name
        assert kvq.kvq_get_state(h) == (4, 128)
    # counters
    for bad in [(-1, 0), (5, 0), (0, 129), (0, -1)]:
        with pytest.raises(kvq.KvqError):
            kvq.kvq_set_state(h, *bad)
    assert kvq.kvq_get_state(h) == (4, 128)
    kvq.kvq_quantize_page(h, FAKE, FAKE, 0, 0)  # zero pages: a no-op
    kvq.kvq_cache_destroy(h)


def test_offsets_follow_the_layout(kvq):
    h, c = _handle(kvq)
    pb = kvq.kvq_page_bytes(c)
    assert kvq.kvq_page_offset(h, 1, 1, 2) == ((1 * 2 + 1) * 4 + 2) * pb
    base = 2 * 2 * 4 * pb
    ko, vo = kvq.kvq_residual_offset(h, 1, 0)
    assert ko == base + 2 * 2 * 128 * 128 * 2 and vo == ko + 128 * 128 * 2
    with pytest.raises(kvq.KvqError):
        kvq.kvq_page_offset(h, 2, 0, 0)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_page_offset(h, 0, 0, 4)
    kvq.kvq_cache_destroy(h)


def test_decode_split_choice(kvq):
    h, c = _handle(kvq, max_pages=64)
    kvq.kvq_set_state(h, 63, 128)
    auto = kvq.kvq_get_decode_splits(h)
    groups = 4 * 63  # runs of 32-token page groups, four runs (waves) per split
    NW = 4
    assert 1 <= auto <= min(-(-groups // NW), 256)
    for s, want in [(1, 1), (7, 7), (20, 20), (63, 63), (100, 63), (1000, 63)]:
        kvq.kvq_set_decode_splits(h, s)
        got = kvq.kvq_get_decode_splits(h)
        # groups per run = ceil(252 / (4 s)); splits = ceil(252 / (4 run))
        run = -(-groups // (NW * want))
        assert got == -(-groups // (NW * run))
    kvq.kvq_set_decode_splits(h, 0)
    assert kvq.kvq_get_decode_splits(h) == auto
    kvq.kvq_cache_destroy(h)


def test_quantize_groups_argument_checks(kvq):
    for args in [(2, 3), (0, 7)]:
        with pytest.raises(kvq.KvqError):
            kvq.kvq_quantize_groups(args[0], args[1], FAKE, 1, 4, FAKE, FAKE, FAKE, 0)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_quantize_groups(0, 3, FAKE, 1, 257, FAKE, FAKE, FAKE, 0)
    kvq.kvq_quantize_groups(0, 3, FAKE, 0, 4, FAKE, FAKE, FAKE, 0)  # no groups: no-op


def test_strerror(kvq):
    for code in range(-7, 1):
        assert kvq.kvq_strerror(code)


# -- block pool ------------------------------------------------------------------
def _pool(kvq, n_blocks=12, **kw):
    c = _cfg(kvq, **kw)
    return kvq.kvq_pool_create(c, n_blocks, FAKE, kvq.kvq_pool_bytes(c, n_blocks)), c


def test_pool_layout_and_limits(kvq):
    c = _cfg(kvq, batch=3, max_pages=5)
    pb = kvq.kvq_page_bytes(c)
    n = kvq.kvq_pool_bytes(c, 7)
    h = kvq.kvq_pool_create(c, 7, FAKE, n)
    try:
        assert kvq.kvq_pool_page_offset(h, 0, 0) == 0
        assert kvq.kvq_pool_page_offset(h, 6, 1) == (6 * 2 + 1) * pb
        ko, vo = kvq.kvq_pool_window_offset(h, 2, 1)
        wbase = (7 * 2 * pb + 255) // 256 * 256
        assert ko == wbase + (2 * 2 + 1) * 2 * 128 * 128 * 2 and vo == ko + 128 * 128 * 2
        t = kvq.kvq_pool_table_offset(h)
        assert t % 256 == 0 and t >= wbase + 3 * 2 * 2 * 128 * 128 * 2
        assert n == t + 3 * 5 * 4
        assert kvq.kvq_pool_free_blocks(h) == 7
        assert kvq.kvq_pool_get_seq(h, 2) == (False, 0, 0)
        for bad in [(7, 0), (-1, 0), (0, 2)]:
            with pytest.raises(kvq.KvqError):
                kvq.kvq_pool_page_offset(h, *bad)
    finally:
        kvq.kvq_pool_destroy(h)
    for bad in [dict(batch=257), dict(max_pages=65536), dict(num_kv_heads=64, num_q_heads=64)]:
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_pool_bytes(_cfg(kvq, **bad), 4)
        assert e.value.name == "KVQ_EINVAL"
    with pytest.raises(kvq.KvqError):
        kvq.kvq_pool_bytes(c, 0)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_pool_create(c, 7, FAKE + 8, n)
    assert e.value.name == "KVQ_EALIGN"
    with pytest.raises(kvq.KvqError):
        kvq.kvq_pool_create(c, 7, FAKE, n - 1)


def test_pool_call_errors_leave_state(kvq):
    h, c = _pool(kvq, n_blocks=3)
    try:
        def code(f):
            with pytest.raises(kvq.KvqError) as e:
                f()
            return e.value.name
        # more pages than max_pages (4) or than free blocks (3): nothing launched
        assert code(lambda: kvq.kvq_pool_prefill(h, 0, FAKE, FAKE, 5 * 128, stream=0)) == \
            "KVQ_ECAPACITY"
        assert code(lambda: kvq.kvq_pool_prefill(h, 0, FAKE, FAKE, 4 * 128, stream=0)) == \
            "KVQ_ECAPACITY"
        assert code(lambda: kvq.kvq_pool_prefill(h, 2, FAKE, FAKE, 1, stream=0)) == "KVQ_EINVAL"
        assert code(lambda: kvq.kvq_pool_prefill(h, 0, FAKE, FAKE, -1, stream=0)) == "KVQ_EINVAL"
        assert code(lambda: kvq.kvq_pool_prefill(h, 0, FAKE + 8, FAKE, 1, stream=0)) == \
            "KVQ_EALIGN"
        assert code(lambda: kvq.kvq_pool_release(h, 0)) == "KVQ_ESTATE"
        assert code(lambda: kvq.kvq_pool_block_of(h, 0, 0)) == "KVQ_EINVAL"
        ws = kvq.kvq_pool_decode_workspace_bytes(h)
        assert code(lambda: kvq.kvq_pool_decode_attention(h, FAKE, FAKE, FAKE, ws - 1,
                                                          stream=0)) == "KVQ_EWORKSPACE"
        assert code(lambda: kvq.kvq_pool_append_decode(h, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1,
                                                       stream=0)) == "KVQ_EWORKSPACE"
        assert code(lambda: kvq.kvq_pool_append(h, FAKE, FAKE + 4, stream=0)) == "KVQ_EALIGN"
        assert kvq.kvq_pool_free_blocks(h) == 3
        assert kvq.kvq_pool_get_seq(h, 0) == (False, 0, 0)
        with pytest.raises(kvq.KvqError):
            kvq.kvq_pool_set_kernel_events(h, FAKE, None)
    finally:
        kvq.kvq_pool_destroy(h)


def test_prefill_argument_checks():
    """kvq_prefill_select rejects bad shapes, budgets, pointers, alignment and
    short workspaces before launching anything; the workspace grows with T."""
    from bit_mixed_precision_page_amd import kvq

    def code(f):
        with pytest.raises(kvq.KvqError) as e:
            f()
        return e.value.name

    ws = kvq.kvq_prefill_workspace_bytes(300, 8, 2)
    assert ws >= 8 * 300 * 4 + 2 * 128 * 320 * 2
    assert kvq.kvq_prefill_workspace_bytes(301, 8, 2) >= ws
    for T, hq, hkv in [(0, 8, 2), ((1 << 20) + 1, 8, 2), (300, 6, 4), (300, 34, 2), (300, 2, 4)]:
        assert code(lambda: kvq.kvq_prefill_workspace_bytes(T, hq, hkv)) == "KVQ_EINVAL"

    def call(dtype=1, T=300, heavy=10, recent=10, q=FAKE, keep=FAKE, k_sel=FAKE, v_sel=FAKE,
             wsb=ws):
        return kvq.kvq_prefill_select(dtype, T, 8, 2, 0.0, q, FAKE, FAKE, heavy, recent, FAKE,
                                      FAKE, keep, k_sel, v_sel, FAKE, wsb, stream=0)
    assert code(lambda: call(dtype=7)) == "KVQ_EINVAL"
    assert code(lambda: call(T=0)) == "KVQ_EINVAL"
    assert code(lambda: call(heavy=-1)) == "KVQ_EINVAL"
    assert code(lambda: call(recent=-1)) == "KVQ_EINVAL"
    assert code(lambda: call(q=None)) == "KVQ_EINVAL"
    assert code(lambda: call(keep=None)) == "KVQ_EINVAL"
    assert code(lambda: call(k_sel=None)) == "KVQ_EINVAL"
    assert code(lambda: call(q=FAKE + 8)) == "KVQ_EALIGN"
    assert code(lambda: call(keep=FAKE + 4)) == "KVQ_EALIGN"
    assert code(lambda: call(wsb=ws - 1)) == "KVQ_EWORKSPACE"
    # timing hooks: both or neither
    assert code(lambda: kvq.kvq_prefill_set_kernel_events(FAKE, None)) == "KVQ_EINVAL"
    kvq.kvq_prefill_set_kernel_events(None, None)


def test_prefill_workspace_covers_the_key_split():
    """Short sequences split the keys and need room for the per-chunk partials
    (m, l and 128 accumulators per row and chunk); long ones do not."""
    from bit_mixed_precision_page_amd import kvq

    def base(T, hq, hkv):
        t32 = (T + 31) // 32 * 32
        return hq * T * 4 + hkv * 16 * T * 4 + hkv * 128 * t32 * 2

    # 1024 tokens, 32 / 8 heads: 256 attention workgroups -> three key chunks
    ws = kvq.kvq_prefill_workspace_bytes(1024, 32, 8)
    assert ws >= base(1024, 32, 8) + 32 * 1024 * 3 * (2 + 128) * 4
    # 8192 tokens: 2048 workgroups, no split, no partials
    ws = kvq.kvq_prefill_workspace_bytes(8192, 32, 8)
    assert base(8192, 32, 8) <= ws < base(8192, 32, 8) + 4 * 256


def test_prefill_key_split_cap_checks(kvq):
    """kvq_prefill_set_max_key_splits accepts 0 (automatic) to 4 and rejects
    anything else without changing the setting."""
    for n in (-1, 5, 100):
        with pytest.raises(kvq.KvqError):
            kvq.kvq_prefill_set_max_key_splits(n)
    for n in (1, 4, 0):
        kvq.kvq_prefill_set_max_key_splits(n)
