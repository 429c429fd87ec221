"""GPU path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars: page bytes, window bytes, quantizer outputs and channel selections are
bit-exact; attention is within max-abs 1e-3 of the oracle's fp64 attention
over the same dequantized cache.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from bit_mixed_precision_page_amd import inputs as gen
from gpu_util import GUARDS, Pair, dev, first_page_mismatch, guarded_cache, host

pytestmark = pytest.mark.gpu
TOL = 1e-3
W = gen.WORKLOADS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_pages(pair):
    g = pair.pages()
    o = pair.ora.pages
    msg = first_page_mismatch(g[:, :, :pair.ora.n_pages], o[:, :, :pair.ora.n_pages])
    assert msg is None, msg
    kw, vw = pair.windows()
    n = pair.ora.n_res
    assert (kw[:, :, :n] == pair.ora.kres[:, :, :n]).all()
    assert (vw[:, :, :n] == pair.ora.vres[:, :, :n]).all()


def check_attention(pair, q, splits=0, tol=TOL):
    got = pair.attention(q, splits)
    ref = pair.ora.attention(q)
    err = np.abs(got - ref).max()
    say(f"    max |gpu - oracle| = {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= tol, f"max abs error {err}"
    return got


def test_quantize_groups_every_range(ora):
    """Device quantizer vs the oracle on groups whose maximum runs over every
    positive finite pattern of each dtype (so every reachable scale and its
    IEEE reciprocal is exercised), for L = 3 and 15."""
    from bit_mixed_precision_page_amd import kvq
    r = np.random.default_rng(99)
    for dt in (gen.F16, gen.BF16):
        bits = np.arange(1, 0x7C00 if dt == gen.F16 else 0x7F80, dtype=np.uint16)
        M = gen.from_bits(bits, dt).astype(np.float64)
        n, glen = len(bits), 8
        frac = r.random((n, glen - 2))
        x = np.concatenate([np.zeros((n, 1)), M[:, None], M[:, None] * frac], axis=1)
        sign = np.where(r.random(n) < 0.3, -1.0, 1.0)[:, None]
        xb = gen.to_bits((x * sign).astype(np.float32), dt)
        for L in (3, 15):
            s = torch.empty(n, dtype=torch.int16, device="cuda")
            z = torch.empty(n, dtype=torch.int16, device="cuda")
            c = torch.empty(n * glen, dtype=torch.uint8, device="cuda")
            kvq.kvq_quantize_groups(dt, L, dev(xb), n, glen, s, z, c)
            torch.cuda.synchronize()
            s, z = host(s).view(np.uint16), host(z).view(np.uint16)
            c = host(c).reshape(n, glen)
            so, zo, co = ora.quantize_groups(dt, xb, L)
            bad = np.flatnonzero((s != so) | (z != zo) | (c != co).any(axis=1))
            assert len(bad) == 0, (dt, L, len(bad), int(bad[0]), xb[bad[0]])
        say(f"  dtype {dt}: all {n} groups bit-exact for L = 3 and 15")


def test_pages_tiny():
    w = W["tiny"]
    pair = Pair(w)
    check_pages(pair)
    check_attention(pair, pair.query())


@pytest.mark.parametrize("name", list(W))
def test_pages_and_attention_reduced(name):
    """Every workload's distribution and dtype at a reduced batch and length."""
    w = W[name]
    pair = Pair(w, B=2, bulk_pages=5, window=37)
    say(f"  {name}: k={pair.k} g={w.g} dtype={w.dtype}")
    check_pages(pair)
    check_attention(pair, pair.query())


def test_append_flush_stream():
    """300 streamed tokens from an empty cache: flushes at tokens 129 and 257."""
    w = dataclasses.replace(W["qwen3_8b_long"], B=2)
    pair = Pair(w, B=2, bulk_pages=0, window=300, max_pages=4)
    assert [i for i, f in enumerate(pair.flushes) if f] == [128, 256]
    assert pair.ora.n_pages == 2 and pair.ora.n_res == 44
    check_pages(pair)
    check_attention(pair, pair.query())


@pytest.mark.parametrize("nres", [1, 77, 128])
def test_window_only(nres):
    pair = Pair(W["llama3_8b_decode"], B=2, bulk_pages=0, window=nres)
    check_attention(pair, pair.query())


def test_pages_only_no_window():
    pair = Pair(W["llama3_8b_decode"], B=2, bulk_pages=3, window=0)
    check_pages(pair)
    check_attention(pair, pair.query())


@pytest.mark.parametrize("boost", [0, 48, 128])
def test_boost_extremes(boost):
    pair = Pair(W["llama3_8b_decode"], B=1, bulk_pages=3, window=5, boost=boost)
    check_pages(pair)
    check_attention(pair, pair.query())


@pytest.mark.parametrize("g", [1, 2, 8, 16])
def test_query_group_sizes(g):
    pair = Pair(W["llama3_8b_decode"], B=1, bulk_pages=2, window=9, Hq=8 * g)
    check_attention(pair, pair.query())


@pytest.mark.parametrize("wl,g,boost", [
    ("llama3_8b_decode", 8, 0), ("llama3_8b_decode", 8, 48), ("llama3_8b_decode", 8, 96),
    ("llama3_8b_decode", 8, 128), ("llama3_8b_decode", 16, 0), ("llama3_8b_decode", 16, 48),
    ("tiny", 8, 16), ("tiny", 16, 32), ("tiny", 2, 80)])
def test_group_size_with_boost_count(wl, g, boost):
    """Each (query group, boosted-channel blocks, dtype) instantiation has its
    own register budget and LDS layout (eight and sixteen heads share the
    K-zero row with the softmax weights): the shapes the workloads do not
    reach, against the oracle."""
    tiny = wl == "tiny"
    pair = Pair(W[wl], B=2, bulk_pages=2, window=33, Hq=(2 if tiny else 8) * g,
                Hkv=2 if tiny else None, boost=boost)
    check_pages(pair)
    check_attention(pair, pair.query())


def test_softmax_scale_argument():
    pair = Pair(W["tiny"], bulk_pages=2, window=3, scale=0.3)
    check_attention(pair, pair.query())


SPLIT_TOL = 1e-4  # split boundaries change the order of fp32 MFMA accumulation (~2e-5 noise)


def test_split_invariance_and_determinism():
    pair = Pair(W["llama3_8b_decode"], B=2, bulk_pages=20, window=100)
    q = pair.query()
    outs = {s: pair.attention(q, s) for s in (1, 3, 7, 20, 0)}
    for s, o in outs.items():
        assert np.abs(o - outs[1]).max() <= SPLIT_TOL, s
    again = pair.attention(q, 0)
    assert (again == outs[0]).all(), "decode attention must be deterministic"
    ref = pair.ora.attention(q)
    assert np.abs(outs[0] - ref).max() <= TOL


def test_snapshot_restore():
    """Pages are position-independent bytes: copy the cache memory into a fresh
    buffer, restore the counters, and the output is bitwise identical."""
    from bit_mixed_precision_page_amd import kvq
    pair = Pair(W["tiny"], bulk_pages=3, window=40, with_oracle=False)
    q = pair.query()
    a = pair.attention(q)
    c2 = guarded_cache(pair.cfg)
    c2.mem.copy_(pair.gpu.mem)
    kvq.kvq_set_state(c2.handle, *pair.gpu.state)
    out = GUARDS.out(pair.B, pair.Hq, 128)
    c2.decode_attention(dev(q), out)
    torch.cuda.synchronize()
    assert (host(out) == a).all()


def test_fused_append_decode_equals_two_calls():
    """kvq_append_decode is kvq_append_token + kvq_decode_attention bit for bit
    (output, page and window bytes), across a window flush; the two-call cache
    follows the oracle."""
    w = W["llama3_8b_decode"]
    fused = Pair(w, B=2, bulk_pages=2, window=126, with_oracle=False)
    ref = Pair(w, B=2, bulk_pages=2, window=126)
    for step in range(4):  # window 127, 128, then flush + 1, 2
        kt, vt = gen.step_kv(w, 500 + step)
        kt, vt = kt[:2], vt[:2]
        q = ref.query(step)
        out = GUARDS.out(2, w.Hq, 128)
        f1 = fused.gpu.append_decode(dev(kt), dev(vt), dev(q), out)
        torch.cuda.synchronize()
        f2 = ref.append(kt, vt)
        assert f1 == f2 == (step == 2)
        assert fused.gpu.state == ref.gpu.state
        got = host(out)
        assert (got == ref.attention(q)).all(), f"step {step}: fused output differs"
        n_pages = ref.ora.n_pages  # pages past the written ones are uninitialized in both
        assert (fused.pages()[:, :, :n_pages] == ref.pages()[:, :, :n_pages]).all()
        kf, vf = fused.windows()
        kr, vr = ref.windows()
        n = ref.ora.n_res
        assert (kf[:, :, :n] == kr[:, :, :n]).all() and (vf[:, :, :n] == vr[:, :, :n]).all()
        check_pages(ref)
        err = np.abs(got - ref.ora.attention(q)).max()
        say(f"    step {step}: fused == two calls; max |gpu - oracle| = {err:.3e}")
        assert err <= TOL
