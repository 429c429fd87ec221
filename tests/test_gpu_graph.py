"""Graph-replayed decode step (kvq_append_decode_device) through the C ABI.

The step's counters live in device memory, so one captured HIP graph serves
every later step.  Every replay is checked against eager calls on a twin cache
fed the same tokens (page and window bytes bit-exact, attention within the
split-count rounding bound) and against the CPU oracle (attention within
max-abs 1e-3), with eager copies and synchronizations between the replays.
"""
import sys

import numpy as np
import pytest
import torch

from bit_mixed_precision_page_amd import inputs as gen
from gpu_util import GUARDS, Pair, assert_plan_ok, dev, host

pytestmark = pytest.mark.gpu
TOL = 1e-3
SPLIT_TOL = 1e-4  # different split counts change only the fp32 summation order
W = gen.WORKLOADS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _compare(graph, ref, out, st, step):
    n_pages, n_res = ref.gpu.state
    got = tuple(host(st)[:2])
    if n_res == 128 and got == (n_pages + 1, 0):
        # the replayed step that filled the window flushed it at its end; the
        # eager twin flushes at the start of its next step (that page is
        # compared then)
        n_res = 0
    else:
        assert got == (n_pages, n_res), f"step {step}: device counters"
    assert host(st)[2] == 0 and host(st)[3] == 0
    assert (graph.pages()[:, :, :n_pages] == ref.pages()[:, :, :n_pages]).all(), \
        f"step {step}: page bytes differ"
    kg, vg = graph.windows()
    kr, vr = ref.windows()
    assert (kg[:, :, :n_res] == kr[:, :, :n_res]).all()
    assert (vg[:, :, :n_res] == vr[:, :, :n_res]).all()


def test_graph_replay_equals_eager_steps():
    w = W["llama3_8b_decode"]
    B = 2
    graph = Pair(w, B=B, bulk_pages=2, window=124, max_pages=5, with_oracle=False)
    ref = Pair(w, B=B, bulk_pages=2, window=124, max_pages=5)
    st = graph.gpu.device_state()
    torch.cuda.synchronize()
    assert tuple(host(st)[:4]) == (2, 124, 0, 0)

    def ref_step(step, kt, vt, q):
        ref.append(kt, vt)
        return ref.attention(q)

    # step 0: the device-counter entry point called eagerly
    kt, vt = gen.step_kv(w, 700)
    kt, vt = kt[:B], vt[:B]
    q = ref.query(0)
    out = GUARDS.out(B, w.Hq, 128)
    assert_plan_ok(graph.gpu, mode=2)
    graph.gpu.append_decode_device(dev(kt), dev(vt), dev(q), out, st)
    torch.cuda.synchronize()
    want = ref_step(0, kt, vt, q)
    assert np.abs(host(out) - want).max() <= SPLIT_TOL
    _compare(graph, ref, out, st, 0)

    # capture one step; its inputs live in static buffers refilled before each replay
    ks = torch.empty(B, w.Hkv, 128, dtype=torch.int16, device="cuda")
    vs = torch.empty_like(ks)
    qs = torch.empty(B, w.Hq, 128, dtype=torch.int16, device="cuda")
    os_ = GUARDS.out(B, w.Hq, 128)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        graph.gpu.append_decode_device(ks, vs, qs, os_, st)
    torch.cuda.synchronize()
    assert tuple(host(st)[:2]) == (2, 125), "capture must not run the step"

    for step in range(1, 9):  # window 126 .. 128 (flushed at the end of step 3), then 1 .. 5
        kt, vt = gen.step_kv(w, 700 + step)
        kt, vt = kt[:B], vt[:B]
        q = ref.query(step)
        ks.copy_(dev(kt))
        vs.copy_(dev(vt))
        qs.copy_(dev(q))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(os_)
        want = ref_step(step, kt, vt, q)
        assert ref.flushes[-1] == (step == 4)
        _compare(graph, ref, os_, st, step)
        d_ref = np.abs(got - want).max()
        d_ora = np.abs(got - ref.ora.attention(q)).max()
        say(f"    replay {step}: state {tuple(int(x) for x in host(st)[:2])}, "
            f"|graph - eager| = {d_ref:.2e}, "
            f"|graph - oracle| = {d_ora:.2e}")
        assert np.isfinite(got).all()
        assert d_ref <= SPLIT_TOL
        assert d_ora <= TOL


def test_graph_step_full_cache_sets_flag():
    """A full window with no free page: the step leaves the cache unchanged,
    skips the token, raises the flag, and attends over the unchanged cache."""
    w = W["llama3_8b_decode"]
    B = 2
    pair = Pair(w, B=B, bulk_pages=2, window=128, max_pages=2)
    pages0 = pair.pages().copy()
    kw0, vw0 = (a.copy() for a in pair.windows())
    st = pair.gpu.device_state()
    kt, vt = gen.step_kv(w, 900)
    q = pair.query(9)
    out = torch.empty(B, w.Hq, 128, dtype=torch.float32, device="cuda")
    pair.gpu.append_decode_device(dev(kt[:B]), dev(vt[:B]), dev(q), out, st)
    torch.cuda.synchronize()
    assert tuple(host(st)[:4]) == (2, 128, 0, 1)
    assert (pair.pages()[:, :, :2] == pages0[:, :, :2]).all()
    kw, vw = pair.windows()
    assert (kw == kw0).all() and (vw == vw0).all()
    err = np.abs(host(out) - pair.ora.attention(q)).max()
    say(f"    full cache: flag set, max |gpu - oracle| = {err:.2e}")
    assert err <= TOL


def test_device_state_init_flushes_a_full_window():
    """A full window with a free page: the state set-up flushes it first (the
    flush the next step would start with), the host counters follow, and a
    replayed step equals the eager step, whose own flush makes the same
    page."""
    w = W["llama3_8b_decode"]
    B = 2
    graph = Pair(w, B=B, bulk_pages=2, window=128, max_pages=4, with_oracle=False)
    ref = Pair(w, B=B, bulk_pages=2, window=128, max_pages=4)
    st = graph.gpu.device_state()
    torch.cuda.synchronize()
    assert tuple(host(st)[:4]) == (3, 0, 0, 0)
    assert graph.gpu.state == (3, 0)
    kt, vt = gen.step_kv(w, 910)
    kt, vt = kt[:B], vt[:B]
    q = ref.query(11)
    out = GUARDS.out(B, w.Hq, 128)
    assert_plan_ok(graph.gpu, mode=2)
    graph.gpu.append_decode_device(dev(kt), dev(vt), dev(q), out, st)
    torch.cuda.synchronize()
    ref.append(kt, vt)
    assert ref.flushes[-1]
    want = ref.attention(q)
    _compare(graph, ref, out, st, 0)
    d_ref = np.abs(host(out) - want).max()
    d_ora = np.abs(host(out) - ref.ora.attention(q)).max()
    say(f"    flushed at set-up: |graph - eager| = {d_ref:.2e}, |graph - oracle| = {d_ora:.2e}")
    assert d_ref <= SPLIT_TOL
    assert d_ora <= TOL


def test_several_caches_in_one_graph():
    """Three caches' steps captured in one graph, as a model's decode step
    holds every layer's attention call: each replay equals eager steps on twin
    caches (pages and windows bit-exact) and the oracle, across flushes that
    fall at different replays for the three caches."""
    w = W["llama3_8b_decode"]
    B = 2
    wins = (124, 127, 60)
    graphs = [Pair(w, B=B, bulk_pages=2, window=n, max_pages=5, with_oracle=False) for n in wins]
    refs = [Pair(w, B=B, bulk_pages=2, window=n, max_pages=5) for n in wins]
    sts = [gp.gpu.device_state() for gp in graphs]
    ins = [(torch.empty(B, w.Hkv, 128, dtype=torch.int16, device="cuda"),
            torch.empty(B, w.Hkv, 128, dtype=torch.int16, device="cuda"),
            torch.empty(B, w.Hq, 128, dtype=torch.int16, device="cuda"),
            GUARDS.out(B, w.Hq, 128)) for _ in wins]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for gp, st, (ks, vs, qs, os_) in zip(graphs, sts, ins):
            gp.gpu.append_decode_device(ks, vs, qs, os_, st)
    torch.cuda.synchronize()
    for step in range(1, 7):
        wants = []
        for i, (ref, (ks, vs, qs, os_)) in enumerate(zip(refs, ins)):
            kt, vt = gen.step_kv(w, 900 + 10 * i + step)
            kt, vt = kt[:B], vt[:B]
            q = ref.query(100 * i + step)
            ks.copy_(dev(kt))
            vs.copy_(dev(vt))
            qs.copy_(dev(q))
            ref.append(kt, vt)
            wants.append((ref.attention(q), ref.ora.attention(q)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (gp, ref, st, (_, _, _, os_)) in enumerate(zip(graphs, refs, sts, ins)):
            got = host(os_)
            _compare(gp, ref, os_, st, step)
            d_ref = np.abs(got - wants[i][0]).max()
            d_ora = np.abs(got - wants[i][1]).max()
            say(f"    replay {step}, cache {i}: state {tuple(int(x) for x in host(st)[:2])}, "
                f"|graph - eager| = {d_ref:.2e}, |graph - oracle| = {d_ora:.2e}")
            assert np.isfinite(got).all()
            assert d_ref <= SPLIT_TOL
            assert d_ora <= TOL
    # the 127-token cache flushed at the end of replay 1, the 124-token one at the end of replay 4
    assert refs[1].flushes[-6:].count(True) == 1 and refs[0].flushes[-6:].count(True) == 1
    assert refs[2].flushes[-6:].count(True) == 0
