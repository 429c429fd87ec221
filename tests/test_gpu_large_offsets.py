"""Caches whose byte offsets do not fit in 32 bits, through the C ABI against
the CPU oracle: every kernel addresses pages, windows and the block table with
64-bit offsets.

Dense cache: two (sequence, KV head) units with room for 2^19 pages each, so
the second unit's pages start 6.7 GB in and both windows sit past 13.4 GB.
Block pool: 180 000 blocks, so every window and the block table lie past
4.6 GB (blocks are handed out from the low end).  Only the written regions
are read back.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from bit_mixed_precision_page_amd import inputs as gen
from gpu_util import GUARDS, Pair, assert_plan_ok, dev, first_page_mismatch, host
from test_gpu_pool import PoolPair

pytestmark = pytest.mark.gpu
TOL = 1e-3
GIB4 = 1 << 32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_dense_cache_beyond_4gib():
    w = gen.WORKLOADS["llama3_8b_decode"]
    mp = 1 << 19
    # 2 bulk pages, then 130 appended tokens: a flush at the 129th
    pair = Pair(w, B=1, Hq=8, Hkv=2, bulk_pages=2, window=130, max_pages=mp)
    pb = pair.gpu.page_bytes
    assert pb * mp > GIB4 // 2 and 2 * pb * mp > 3 * GIB4  # unit 1 past 4 GiB, windows past 12 GiB
    say(f"  cache {pair.gpu.nbytes / 1e9:.1f} GB, page area {2 * pb * mp / 1e9:.1f} GB")
    assert pair.flushes.count(True) == 1
    o = pair.ora
    n = o.n_pages
    torch.cuda.synchronize()
    got = host(pair.gpu.pages_view()[:, :, :n])
    msg = first_page_mismatch(got, o.pages[:, :, :n])
    assert msg is None, msg
    kw, vw = pair.windows()
    assert (kw[:, :, :o.n_res] == o.kres[:, :, :o.n_res]).all()
    assert (vw[:, :, :o.n_res] == o.vres[:, :, :o.n_res]).all()
    q = pair.query()
    got = pair.attention(q)
    err = float(np.abs(got - o.attention(q)).max())
    say(f"    attention: max |gpu - oracle| = {err:.3e}")
    assert err <= TOL
    # the fused step (window slot written by the split kernel past 13.4 GB)
    out = GUARDS.out(1, 8, 128)
    for step in range(3):
        r = np.random.default_rng(700 + step)
        k = gen.to_bits(r.standard_normal((1, 2, 128), dtype=np.float32), w.dtype)
        v = gen.to_bits(r.standard_normal((1, 2, 128), dtype=np.float32), w.dtype)
        q = gen.to_bits(r.standard_normal((1, 8, 128), dtype=np.float32), w.dtype)
        assert_plan_ok(pair.gpu, mode=1)
        pair.gpu.append_decode(dev(k), dev(v), dev(q), out)
        o.append(k, v)
        torch.cuda.synchronize()
        err = float(np.abs(host(out) - o.attention(q)).max())
        say(f"    fused step {step}: max |gpu - oracle| = {err:.3e}")
        assert err <= TOL
    kw, vw = pair.windows()
    assert (kw[:, :, :o.n_res] == o.kres[:, :, :o.n_res]).all()
    assert (vw[:, :, :o.n_res] == o.vres[:, :, :o.n_res]).all()


def test_pool_windows_and_table_beyond_4gib():
    w = dataclasses.replace(gen.WORKLOADS["tiny"], B=3, Hq=8, Hkv=2, boost=16, dtype=gen.BF16)
    n_blocks = 180000
    pair = PoolPair(w, n_blocks=n_blocks, max_pages=8)
    assert n_blocks * w.Hkv * pair.gpu.page_bytes > GIB4
    pair.prefill(0, 300)
    pair.prefill(2, 129)
    pair.check_state()
    out = GUARDS.out(w.B, w.Hq, 128)
    for step in range(1, 131):
        k, v, q = pair.step_inputs(step)
        nf = pair.gpu.append(dev(k), dev(v))
        assert nf == pair.oracle_append(k, v), step
        if step in (1, 128, 130):
            pair.check_state()
            assert_plan_ok(pair.gpu)
            pair.gpu.decode_attention(dev(q), out)
            torch.cuda.synchronize()
            err = pair.check_attention(host(out), q)
            say(f"    pool step {step}: max |gpu - oracle| = {err:.3e}")
