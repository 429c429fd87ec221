"""Query-aware Key channel ranking (MixKVQ abstract: difficulty x relevance)
through the C ABI against the CPU oracle: relevance vectors bit-exact, every
page quantized with a relevance vector bit-exact (bulk, window flushes, block
pool), attention over such pages within max-abs 1e-3 of the fp64 oracle."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from bit_mixed_precision_page_amd import inputs as gen
from gpu_util import Pair, dev, first_page_mismatch, guarded_pool, host

pytestmark = pytest.mark.gpu
P = 128
TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dt,B,Hq,Hkv", [(gen.F16, 3, 8, 8), (gen.BF16, 5, 32, 8),
                                         (gen.BF16, 2, 16, 2), (gen.F16, 1, 4, 1)])
def test_query_relevance_bit_exact(ora, dt, B, Hq, Hkv):
    from bit_mixed_precision_page_amd import kvq
    r = np.random.default_rng(B * 100 + Hq)
    q = gen.to_bits(r.standard_normal((B, Hq, 128), dtype=np.float32) *
                    np.exp(r.uniform(-3, 3, (1, 1, 128))).astype(np.float32), dt)
    out = torch.empty(B, Hkv, 128, dtype=torch.float32, device="cuda")
    kvq.kvq_query_relevance(dt, B, Hq, Hkv, dev(q), out)
    torch.cuda.synchronize()
    ref = ora.query_relevance(dt, q, Hkv)
    assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name,boost", [("tiny", 16), ("llama3_8b_decode", 32)])
def test_query_aware_dense_pages(ora, name, boost):
    """Bulk pages and streamed flushes with a relevance vector (from the
    step's query) bit-exact; the selections differ from the magnitude
    ranking's on some pages; attention within tolerance."""
    w = dataclasses.replace(gen.WORKLOADS[name], B=min(gen.WORKLOADS[name].B, 2))
    pair = Pair(w, B=w.B, bulk_pages=0, window=0, boost=boost, max_pages=5)
    q0 = pair.query(step=0)
    rel = ora.query_relevance(w.dtype, q0, pair.Hkv)
    rel_d = torch.from_numpy(rel).cuda()
    pair.gpu.set_relevance(rel_d)
    pair.ora.rel = rel
    T = 2 * P
    K, V = gen.prefill_kv(dataclasses.replace(w, Hkv=pair.Hkv, Hq=pair.Hq), ntok=T + P + 9)
    pair.gpu.quantize_page(dev(np.ascontiguousarray(K[:, :, :T])),
                           dev(np.ascontiguousarray(V[:, :, :T])), 2)
    pair.ora.quantize_pages(K[:, :, :T], V[:, :, :T])
    for t in range(T, T + P + 9):
        pair.append(K[:, :, t], V[:, :, t])
    assert pair.ora.n_pages == 3 and pair.ora.n_res == 9
    g = pair.pages()
    msg = first_page_mismatch(g[:, :, :3], pair.ora.pages[:, :, :3])
    assert msg is None, msg
    # the relevance changed the choice somewhere
    lay = ora.page_layout(boost)
    differs = 0
    for b in range(w.B):
        for h in range(pair.Hkv):
            for p in range(3):
                src = K[b, h, p * P:(p + 1) * P]
                _, idx_mag = ora.select_channels(src, boost)
                idx = g[b, h, p, lay["kidx"]:lay["kidx"] + boost]
                differs += int(not np.array_equal(idx, idx_mag))
    say(f"    {differs} of {w.B * pair.Hkv * 3} pages chose other channels than the magnitude ranking")
    assert differs > 0
    got = pair.attention(q0)
    err = np.abs(got - pair.ora.attention(q0)).max()
    say(f"    attention max |gpu - oracle| = {err:.3e}")
    assert err <= TOL


def test_query_aware_pool_pages(ora):
    """Block pool: prefill and flushes with per-sequence relevance rows."""
    from bit_mixed_precision_page_amd import kvq
    w = dataclasses.replace(gen.WORKLOADS["tiny"], B=4, Hq=8, Hkv=2, dtype=gen.BF16)
    cfg = kvq.config(w.B, w.Hq, w.Hkv, 16, 8, w.dtype)
    pool = guarded_pool(cfg, 24)
    r = np.random.default_rng(77)
    rel = np.abs(r.standard_normal((w.B, w.Hkv, 128))).astype(np.float32)
    rel[1] = 0.0
    rel[1, :, 5:21] = 1.0  # sequence 1: relevance only on channels 5..20
    rel_d = torch.from_numpy(rel).cuda()
    pool.set_relevance(rel_d)
    lengths = {0: 300, 1: 200, 3: 127}
    ref = {}
    for s, n in lengths.items():
        K = np.empty((w.Hkv, n, 128), np.uint16)
        V = np.empty_like(K)
        for h in range(w.Hkv):
            K[h], V[h] = gen.unit_kv(w, s, h, n)
        pool.prefill(s, dev(K), dev(V))
        o = oracle.OracleCache(w.dtype, 1, w.Hq, w.Hkv, 16, 8)
        o.rel = rel[s:s + 1]
        full = n // P
        if full:
            o.quantize_pages(K[None, :, :full * P], V[None, :, :full * P])
        for t in range(full * P, n):
            o.append(K[None, :, t], V[None, :, t])
        ref[s] = o
    for step in range(1, 60):
        k = gen.to_bits(r.standard_normal((w.B, w.Hkv, 128), dtype=np.float32), w.dtype)
        v = gen.to_bits(r.standard_normal((w.B, w.Hkv, 128), dtype=np.float32), w.dtype)
        nf = pool.append(dev(k), dev(v))
        assert nf == sum(int(o.append(k[s:s + 1], v[s:s + 1])) for s, o in ref.items())
    torch.cuda.synchronize()
    lay = ora.page_layout(16)
    for s, o in ref.items():
        live, n_pages, n_res = pool.seq(s)
        assert (n_pages, n_res) == (o.n_pages, o.n_res)
        for p in range(n_pages):
            blk = pool.block_of(s, p)
            for h in range(w.Hkv):
                got = host(pool.page_view(blk, h))
                assert np.array_equal(got, o.pages[0, h, p]), (s, p, h)
                if s == 1:
                    idx = got[lay["kidx"]:lay["kidx"] + 16]
                    assert idx.tolist() == list(range(5, 21))
    say(f"    pool pages with relevance bit-exact ({sum(pool.seq(s)[1] for s in ref)} per head)")


def test_query_aware_graph_step_flush(ora):
    """The merge launch of a graph-replayable step flushes the window its step
    filled with the cache's relevance vector: that page bit-exact with the
    oracle's, and attention after the flush within tolerance."""
    w = dataclasses.replace(gen.WORKLOADS["llama3_8b_decode"], B=2)
    graph = Pair(w, B=2, bulk_pages=1, window=126, max_pages=4, with_oracle=False)
    ref = Pair(w, B=2, bulk_pages=1, window=126, max_pages=4)
    rel = ora.query_relevance(w.dtype, ref.query(step=0), ref.Hkv)
    rel_d = torch.from_numpy(rel).cuda()
    graph.gpu.set_relevance(rel_d)
    ref.gpu.set_relevance(rel_d)
    ref.ora.rel = rel
    st = graph.gpu.device_state()
    out = torch.empty(2, w.Hq, 128, dtype=torch.float32, device="cuda")
    for step in range(3):  # window 127, 128 (flushed by that step's merge launch), then 1
        kt, vt = gen.step_kv(w, 300 + step)
        kt, vt = kt[:2], vt[:2]
        q = ref.query(step)
        graph.gpu.append_decode_device(dev(kt), dev(vt), dev(q), out, st)
        ref.append(kt, vt)
    torch.cuda.synchronize()
    assert tuple(host(st)[:4]) == (2, 1, 0, 0)
    assert ref.ora.n_pages == 2 and ref.ora.n_res == 1 and ref.flushes[-1]
    msg = first_page_mismatch(graph.pages()[:, :, :2], ref.ora.pages[:, :, :2])
    assert msg is None, msg
    err = np.abs(host(out) - ref.ora.attention(q)).max()
    say(f"    graph step with relevance: flushed page bit-exact, max |gpu - oracle| = {err:.3e}")
    assert err <= TOL
