"""Every workload at its full size, in the launch configuration the benchmark
times (automatic split choice), through the C ABI.

Page bytes and window bytes are compared with the oracle for every page of
every (sequence, KV head) unit: the oracle quantizes the same inputs page by
page, in threads.  Attention is compared with the oracle's fp64 attention over
its own pages and the input window tokens on every (sequence, KV head) unit of
every workload.  The long-context streaming workload runs its
256 decode steps: every step's output must be finite, and steps 1, 128, 129
(the step after the window flush) and 256 are compared with the oracle.
"""
import concurrent.futures as cf
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from bit_mixed_precision_page_amd import inputs as gen
from gpu_util import GUARDS, assert_plan_ok, dev, guarded_cache, host

pytestmark = pytest.mark.gpu
P = 128
TOL = 1e-3
THREADS = max(1, min(16, os.cpu_count() or 1))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build_gpu(w, K, V, bulk, window):
    from bit_mixed_precision_page_amd import kvq
    cfg = kvq.config(w.B, w.Hq, w.Hkv, w.boost, w.max_pages, w.dtype)
    c = guarded_cache(cfg)
    if bulk:
        c.quantize_page(dev(K[:, :, :bulk * P]), dev(V[:, :, :bulk * P]), bulk)
    for t in range(window):
        c.append_token(dev(K[:, :, bulk * P + t]), dev(V[:, :, bulk * P + t]))
    torch.cuda.synchronize()
    return c


def oracle_pages(w, K, V, n_pages, max_pages):
    """The oracle's page bytes [B][Hkv][max_pages][page bytes] from the inputs,
    quantized page by page in threads (each unit independently)."""
    ora = oracle.lib()
    pages = np.zeros((w.B, w.Hkv, max_pages, ora.page_bytes(w.boost)), np.uint8)

    def unit(bh):
        b, h = bh
        for p in range(n_pages):
            sl = slice(p * P, (p + 1) * P)
            pages[b, h, p], _, _ = ora.quantize_page(w.dtype, w.boost, K[b, h, sl], V[b, h, sl])

    with cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(unit, [(b, h) for b in range(w.B) for h in range(w.Hkv)]))
    return pages


def assert_pages_equal(ref, got, n_pages):
    bad = np.argwhere((ref[:, :, :n_pages] != got[:, :, :n_pages]).any(axis=-1))
    if len(bad):
        b, h, p = bad[0]
        byte = int(np.flatnonzero(ref[b, h, p] != got[b, h, p])[0])
        raise AssertionError(f"{len(bad)} pages differ; first unit ({b},{h}) page {p} byte {byte}")


def oracle_attention(w, pages, kres, vres, q, n_pages, n_res, units):
    """fp64 attention of the oracle over its own pages and the input window
    tokens, for units [u0, u1)."""
    scale = 1.0 / np.sqrt(128.0)
    return oracle.lib().attention(w.dtype, w.boost, pages, kres, vres, q, n_pages, n_res,
                                  scale, units=units)


def gpu_attention(gpu, q, w):
    out = GUARDS.out(w.B, w.Hq, 128)
    assert_plan_ok(gpu)
    gpu.decode_attention(dev(q), out)
    torch.cuda.synchronize()
    return host(out)


def compare(got, ref, w, units):
    u0, u1 = units
    g = w.g
    rows = []
    for u in range(u0, u1):
        b, h = divmod(u, w.Hkv)
        rows.append((b, slice(h * g, (h + 1) * g)))
    err = max(np.abs(got[b, hs] - ref[b, hs]).max() for b, hs in rows)
    assert np.isfinite(got).all()
    return err


@pytest.mark.parametrize("name,units", [
    ("tiny", None), ("llama3_8b_decode", None), ("qwen3_8b_long", None),
    ("llama70b_large_batch", None),
])
def test_full_size_state(name, units):
    w = gen.WORKLOADS[name]
    bulk, window = w.prefill_pages, w.prefill_residual
    say(f"  {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} ctx={bulk * P + window} k={w.boost}")
    K, V = gen.prefill_kv(w, ntok=bulk * P + window)
    gpu = build_gpu(w, K, V, bulk, window)
    n_pages, n_res = gpu.state
    assert (n_pages, n_res) == (bulk, window)
    pages = oracle_pages(w, K, V, n_pages, w.max_pages)
    assert_pages_equal(pages, host(gpu.pages_view()), n_pages)
    kres = np.zeros((w.B, w.Hkv, P, 128), np.uint16)
    vres = np.zeros_like(kres)
    kres[:, :, :n_res], vres[:, :, :n_res] = K[:, :, bulk * P:], V[:, :, bulk * P:]
    kw, vw = gpu.window_view()
    assert np.array_equal(host(kw).view(np.uint16)[:, :, :n_res], kres[:, :, :n_res])
    assert np.array_equal(host(vw).view(np.uint16)[:, :, :n_res], vres[:, :, :n_res])
    say(f"    all {w.B * w.Hkv * n_pages} pages and the windows bit-exact")
    q = gen.query(w)
    got = gpu_attention(gpu, q, w)
    units = units or (0, w.B * w.Hkv)
    ref = oracle_attention(w, pages, kres, vres, q, n_pages, n_res, units)
    err = compare(got, ref, w, units)
    say(f"    units {units}: max |gpu - oracle| = {err:.3e}")
    assert err <= TOL


def test_long_prefill_then_decode_steps():
    w = gen.WORKLOADS["long_prefill_decode"]
    bulk = w.prefill_pages
    say(f"  prefill {bulk} pages x {w.B * w.Hkv} units, then {w.decode_steps} steps")
    K, V = gen.prefill_kv(w, ntok=bulk * P)
    gpu = build_gpu(w, K, V, bulk, 0)
    pages = oracle_pages(w, K, V, bulk, w.max_pages)
    assert_pages_equal(pages, host(gpu.pages_view()), bulk)
    say("    prefill pages bit-exact")
    ora = oracle.lib()
    kres = np.zeros((w.B, w.Hkv, P, 128), np.uint16)
    vres = np.zeros_like(kres)
    n_pages, n_res = bulk, 0
    units = (0, w.B * w.Hkv)
    for s in range(1, w.decode_steps + 1):
        kt, vt = gen.step_kv(w, s)
        flushed = gpu.append_token(dev(kt), dev(vt))
        if n_res == P:  # flush-before-insert: the full window becomes a page
            assert flushed
            for b in range(w.B):
                for h in range(w.Hkv):
                    pages[b, h, n_pages], _, _ = ora.quantize_page(w.dtype, w.boost, kres[b, h],
                                                                   vres[b, h])
            assert_pages_equal(pages, host(gpu.pages_view()), n_pages + 1)
            n_pages, n_res = n_pages + 1, 0
            say(f"    step {s}: flushed window page bit-exact")
        else:
            assert not flushed
        kres[:, :, n_res], vres[:, :, n_res] = kt, vt
        n_res += 1
        assert gpu.state == (n_pages, n_res)
        q = gen.query(w, step=s)
        got = gpu_attention(gpu, q, w)
        assert np.isfinite(got).all(), s
        if s in (1, 128, 129, 256):
            kw, vw = gpu.window_view()
            assert np.array_equal(host(kw).view(np.uint16)[:, :, :n_res], kres[:, :, :n_res])
            assert np.array_equal(host(vw).view(np.uint16)[:, :, :n_res], vres[:, :, :n_res])
            ref = oracle_attention(w, pages, kres, vres, q, n_pages, n_res, units)
            err = compare(got, ref, w, units)
            say(f"    step {s} ({n_pages} pages + {n_res} window): max |gpu - oracle| = {err:.3e}")
            assert err <= TOL
