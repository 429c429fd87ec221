#!/usr/bin/env python3
"""Decode-step benchmark of the 2-bit mixed-precision KV cache on one MI355X.

One step = one decode step of one attention layer: append the new token's K
and V into the window (flushing a full window into a page when needed) and
run split-K decode attention of the new query over the whole cache, through
the fused kvq_append_decode entry point (--unfused: the two separate calls).
Layers rotate over enough independent cache replicas (>= 1 GiB) that every
step reads its cache from HBM, not from the 256 MB Infinity Cache; the
replicas' window fills are staggered so that they flush one at a time, at
the steady-state rate of one flush per 128 steps, whatever the step count.
Inputs are seeded synthetic tensors of the workload's shape, resident in HBM
before the timed region.

Prints one JSON line: value = algorithmic bytes moved by the timed steps /
elapsed time (GB/s); step_us = per-step percentiles (from the split kernel's
own dispatch timestamps on a second run of as many steps), flush steps apart;
graph_step_us = the same step replayed from a captured HIP graph per layer;
graph_all_layers_step_us = per layer step, every layer's step in one graph; roofline =
the split decode kernel's algorithmic bytes per launch / its average launch
time; copy_gbs and read_gbs = the library's bandwidth probe copying and
reading 1 GiB (the measured reference beside the 8 TB/s specification);
cpu_baseline = the CPU oracle on the same cache.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn effective HBM GB/s (packed KV) + tokens/s at 8K ctx, % of HBM peak"
HBM_PEAK_GBS = 8000.0
PAGE = 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_decode")
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9,
                    help="bytes of cache replicas the steps rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="page splits (0 = automatic)")
    ap.add_argument("--event-every", type=int, default=4,
                    help="bracket the split kernel with HIP events on every N-th timed step")
    ap.add_argument("--unfused", action="store_true",
                    help="step = kvq_append_token + kvq_decode_attention (default: the fused "
                         "kvq_append_decode, same results)")
    ap.add_argument("--event-fence", action="store_true",
                    help="events with the default system-scope fence (slower markers)")
    ap.add_argument("--ctx", type=int, default=0,
                    help="decode workloads: context length in tokens, a multiple of 128 "
                         "(0 = the workload's)")
    ap.add_argument("--window", type=int, default=0,
                    help="decode workloads: every replica starts with this many window tokens "
                         "(1..128) instead of the staggered fills")
    ap.add_argument("--tokens", type=int, default=0,
                    help="prefill selection workload: sequence length (0 = the workload's)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the graph-replayed step (kvq_append_decode_device captured once "
                         "per layer replica)")
    ap.add_argument("--lean", action="store_true",
                    help="headline phase only (no per-step timestamps, graph step, bandwidth "
                         "probes or CPU baseline): the run a profiler wraps")
    ap.add_argument("--query-aware", action="store_true",
                    help="rank Key channels by group range x query relevance (relevance of "
                         "the first decode query) instead of magnitude")
    return ap.parse_args()


def attention_bytes(w, k_page_bytes, n_pages, n_res):
    """Algorithmic bytes of one decode-attention call: every packed page, every
    window token (K and V), the query and the fp32 output."""
    units = w.B * w.Hkv
    return (units * (n_pages * k_page_bytes + n_res * 2 * 128 * 2) + w.B * w.Hq * 128 * 2 +
            w.B * w.Hq * 128 * 4)


def append_bytes(w, k_page_bytes, flushed):
    """Append: read the token's K and V, write them into the window; a flush
    also reads the 128-token window and writes one page."""
    units = w.B * w.Hkv
    b = units * 2 * 128 * 2 * 2
    if flushed:
        b += units * (128 * 128 * 2 * 2 + k_page_bytes)
    return b


def pmc_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__pmc.txt")
    if not os.path.exists(path):
        return None
    from bit_mixed_precision_page_amd.profsum import source_sha256
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_sha256(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


class HipEvents:
    """Timing events created through the HIP runtime with an explicit flag:
    hipEventDisableSystemFence leaves out the system-scope fence when the
    marker completes, which shortens the gap a marker opens in the stream."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n, fence):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        flags = 0 if fence else self.DISABLE_SYSTEM_FENCE
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(flags))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e)

    def pair(self, i):
        return self.ev[2 * i].value, self.ev[2 * i + 1].value

    def elapsed_ms(self, i):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[2 * i], self.ev[2 * i + 1])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value


def staggered_windows(L):
    """Window fill of layer replica i when the timed steps start, spread
    evenly over 1..128 and centred away from a flush: the replicas then flush
    one at a time, about every 128 steps (the steady-state rate), whatever
    the number of timed steps."""
    return [max(1, 128 - (128 * i + 64) // L) for i in range(L)]


def probe_bandwidth(torch, kvq, dev, nbytes, reps=5):
    """The library's bandwidth probe over nbytes of HBM (kvq_probe_bandwidth):
    (copy GB/s counting bytes read + written, read-only GB/s), best of
    `reps` each."""
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    out = []
    for mode, moved in ((1, 2 * nbytes), (0, nbytes)):
        kvq.kvq_probe_bandwidth(mode, src, dst if mode == 1 else sink, nbytes)
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            kvq.kvq_probe_bandwidth(mode, src, dst if mode == 1 else sink, nbytes)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        out.append(moved / (best / 1e3) / 1e9)
    del src, dst
    return out[0], out[1]


def pctl(x):
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return None
    return {"p10": round(float(np.percentile(x, 10)), 2), "p50": round(float(np.median(x)), 2),
            "p90": round(float(np.percentile(x, 90)), 2), "n": int(x.size)}


def dtype_name(gen, w):
    return "bf16" if w.dtype == gen.BF16 else "f16"


def main():
    a = parse()
    if a.lean:
        a.graph, a.no_cpu_baseline = False, True
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the path would shard by (sequence, KV head), with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from bit_mixed_precision_page_amd import inputs as gen
    from bit_mixed_precision_page_amd import kvq

    w = gen.WORKLOADS[a.workload]
    if a.ctx:
        if a.ctx % PAGE or a.ctx < 2 * PAGE:
            raise SystemExit("--ctx must be a multiple of 128 and at least 256")
        import dataclasses
        w = dataclasses.replace(w, ctx=a.ctx)
    if w.decode_steps:
        return stream_main(a, w, torch, gen, kvq)
    if w.ctx_spread:
        return pool_main(a, w, torch, gen, kvq)
    if w.select:
        return prefill_main(a, w, torch, gen, kvq)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    t0 = time.time()
    print(f"[bench] workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} ctx={w.ctx} k={w.boost}",
          file=sys.stderr, flush=True)
    # Cache state: (ctx/128 - 1) bulk pages + a full window of 128 tokens;
    # replica i starts its timed steps with the first n_i of those window
    # tokens (staggered_windows), so the layers reach ctx tokens one after
    # another and flush one at a time.
    bulk = w.ctx // PAGE - 1
    n_win = PAGE
    K, V = gen.prefill_kv(w, ntok=bulk * PAGE + n_win)
    steps_total = a.warmup + 2 * a.steps
    max_pages = w.ctx // PAGE + 1 + (steps_total // PAGE + 2)
    cfg = kvq.config(w.B, w.Hq, w.Hkv, w.boost, max_pages, w.dtype)
    base = kvq.Cache(cfg, device=dev)
    Kd = to_dev(K[:, :, :bulk * PAGE])
    Vd = to_dev(V[:, :, :bulk * PAGE])
    base.quantize_page(Kd, Vd, bulk)
    for t in range(n_win):
        base.append_token(to_dev(K[:, :, bulk * PAGE + t]), to_dev(V[:, :, bulk * PAGE + t]))
    torch.cuda.synchronize()
    del Kd, Vd
    n_pages0, n_res0 = base.state
    assert (n_pages0, n_res0) == (bulk, n_win)
    # (never more replicas than timed steps: a tiny cache is launch-bound anyway)
    layers = min(max(2, math.ceil(a.rotate_bytes / base.nbytes)), max(2, a.steps))
    caches = [base] + [kvq.Cache(cfg, device=dev) for _ in range(layers - 1)]
    snap = base.mem.clone()
    wins = [a.window] * layers if a.window else staggered_windows(layers)

    def restore():
        """Every replica back to the staggered starting state."""
        for c, n in zip(caches, wins):
            c.mem.copy_(snap)
            kvq.kvq_set_state(c.handle, n_pages0, n)
        torch.cuda.synchronize()

    restore()
    if a.splits:
        for c in caches:
            kvq.kvq_set_decode_splits(c.handle, a.splits)
    # Per-step inputs, resident before timing.
    qs, kts, vts = [], [], []
    for s in range(steps_total):
        qs.append(to_dev(gen.query(w, step=s)))
        kt, vt = gen.step_kv(w, s)
        kts.append(to_dev(kt))
        vts.append(to_dev(vt))
    out = torch.empty(w.B, w.Hq, 128, dtype=torch.float32, device=dev)
    timed = [i for i in range(a.steps) if a.event_every > 0 and i % a.event_every == 0]
    hev = HipEvents(len(timed), a.event_fence)
    ev_of = {i: hev.pair(j) for j, i in enumerate(timed)}
    hall = None if a.lean else HipEvents(a.steps, a.event_fence)  # every step's split kernel
    torch.cuda.synchronize()
    print(f"[bench] setup {time.time() - t0:.1f}s; {layers} layer replicas of "
          f"{base.nbytes / 1e6:.1f} MB (replica bytes {base.nbytes}); state {n_pages0} pages + "
          f"windows {wins}", file=sys.stderr, flush=True)

    pb = base.page_bytes

    # Launch arguments as plain integers, resolved once: the loop then costs
    # the host little more than the C calls themselves (a tiny cache is
    # otherwise bound by the Python launch rate, not by the GPU).
    sp = torch.cuda.current_stream().cuda_stream
    kp = [t.data_ptr() for t in kts]
    vp = [t.data_ptr() for t in vts]
    qp = [t.data_ptr() for t in qs]
    op = out.data_ptr()
    hw = [(c.handle, c.ws.data_ptr(), c.ws_bytes) for c in caches]
    host_state = {}

    def reset_host_state():
        for li, c in enumerate(caches):
            host_state[li] = list(c.state)

    def step(s, ev=None):
        li = s % layers
        h, wsp, wsb = hw[li]
        if ev is not None:
            kvq.kvq_set_kernel_events(h, ev[0], ev[1])
        if a.unfused:
            flushed = kvq.kvq_append_token(h, kp[s], vp[s], sp)
            kvq.kvq_decode_attention(h, qp[s], op, wsp, wsb, sp)
        else:
            flushed = kvq.kvq_append_decode(h, kp[s], vp[s], qp[s], op, wsp, wsb, sp)
        if ev is not None:
            kvq.kvq_set_kernel_events(h, None, None)
        st = host_state[li]  # the counters the library keeps, tracked here without a call
        if flushed:
            st[0], st[1] = st[0] + 1, 0
        st[1] += 1
        return flushed, st[0], st[1]

    reset_host_state()
    for s in range(a.warmup):
        step(s)
    torch.cuda.synchronize()
    restore()  # warm-up steps leave no trace in the timed state
    reset_host_state()

    # -- phase 1 (headline): K steps between two events; the split kernel's
    # own dispatch timestamps on every event_every-th step give its duration
    total_bytes = 0
    attn_bytes_sum = 0
    split_bytes = []
    n_flush = 0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    t_host = time.perf_counter()
    for i in range(a.steps):
        s = i  # layer i % layers at its (i // layers)-th visit
        flushed, n_pages, n_res = step(s, ev_of.get(i))
        ab = attention_bytes(w, pb, n_pages, n_res)
        attn_bytes_sum += ab
        total_bytes += ab + append_bytes(w, pb, flushed)
        if i in ev_of:
            split_bytes.append(ab - w.B * w.Hq * 128 * 4)  # pages + window + query
        n_flush += int(flushed)
    end.record()
    host_us = (time.perf_counter() - t_host) / a.steps * 1e6  # launch loop, host side
    torch.cuda.synchronize()
    assert all(tuple(host_state[li]) == caches[li].state for li in range(layers))
    ms = start.elapsed_time(end)
    ms_step = ms / a.steps
    kern_ms = np.array([hev.elapsed_ms(j) for j in range(len(timed))])
    kern_avg_s = float(kern_ms.mean()) / 1e3 if len(timed) else float("nan")
    achieved = float(np.mean(split_bytes)) / kern_avg_s / 1e9 if len(timed) else float("nan")
    value = total_bytes / (ms / 1e3) / 1e9
    attn_gbs = attn_bytes_sum / (ms / 1e3) / 1e9
    splits = kvq.kvq_get_decode_splits(caches[0].handle)
    print(f"[bench] {a.steps} steps in {ms:.3f} ms ({ms_step * 1e3:.1f} us/step, "
          f"split kernel avg {kern_avg_s * 1e6:.1f} us over {len(timed)} launches, "
          f"{n_flush} flushes; host {host_us:.1f} us/step to launch)", file=sys.stderr, flush=True)

    # -- phase 2 (distribution): the next K steps with every split kernel's
    # dispatch timestamps; a step = from one split kernel's start to the
    # next's (its combine, and the next step's flush when there is one)
    step_dist = None
    if not a.lean:
        flush_at = []
        for i in range(a.steps):
            s = a.steps + i
            f, _, _ = step(s, hall.pair(i))
            flush_at.append(bool(f))
        torch.cuda.synchronize()
        assert all(tuple(host_state[li]) == caches[li].state for li in range(layers))
        kern_all = np.array([hall.elapsed_ms(j) for j in range(a.steps)]) * 1e3
        gaps = []
        for i in range(a.steps - 1):
            ms_i = hall.ct.c_float()
            hall.hip.hipEventElapsedTime(hall.ct.byref(ms_i), hall.ev[2 * i], hall.ev[2 * (i + 1)])
            gaps.append(ms_i.value * 1e3)
        gaps = np.array(gaps)
        fl = np.array(flush_at[1:])  # interval i holds the flush of step i + 1
        # (the timestamps themselves widen each step a little: "mean" beside
        # ms_per_step shows by how much)
        step_dist = {"from": "split kernel start to the next step's start, per-step dispatch "
                             "timestamps", "mean": round(float(gaps.mean()), 2),
                     "non_flush": pctl(gaps[~fl]), "flush": pctl(gaps[fl]),
                     "split_kernel": pctl(kern_all[~np.array(flush_at)])}

    # -- graph-replayed step (kvq_append_decode_device captured once per
    # layer replica): the launch-floor comparison
    graph_us = graph_model_us = None
    if not a.unfused and a.graph:
        restore()
        sts = [c.device_state() for c in caches]
        side = torch.cuda.Stream()
        graphs = []
        for li, c in enumerate(caches):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                c.append_decode_device(kts[li % steps_total], vts[li % steps_total],
                                       qs[li % steps_total], out, sts[li])
            graphs.append(g)
        torch.cuda.synchronize()
        for li in range(layers):  # one untimed replay each
            graphs[li].replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for i in range(a.steps):
            graphs[i % layers].replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) / a.steps * 1e3
        err_flags = [int(x.cpu()[3]) for x in sts]
        assert not any(err_flags), "a graph-replayed step found its cache full"
        print(f"[bench] graph-replayed steps: {graph_us:.1f} us/step", file=sys.stderr, flush=True)

        # every layer replica's step in one graph, as a model's decode step
        # would capture its layers' attention calls together: no host launch
        # between layers
        restore()
        sts = [c.device_state() for c in caches]
        gm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gm, stream=side):
            for li, c in enumerate(caches):
                c.append_decode_device(kts[li % steps_total], vts[li % steps_total],
                                       qs[li % steps_total], out, sts[li])
        torch.cuda.synchronize()
        gm.replay()  # untimed
        torch.cuda.synchronize()
        reps = max(1, a.steps // layers)
        g0.record()
        for _ in range(reps):
            gm.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_model_us = g0.elapsed_time(g1) / (reps * layers) * 1e3
        err_flags = [int(x.cpu()[3]) for x in sts]
        assert not any(err_flags), "a graph-replayed step found its cache full"
        print(f"[bench] all {layers} layer steps in one graph: {graph_model_us:.1f} us per layer step "
              f"({reps} replays)", file=sys.stderr, flush=True)

    copy_gbs = read_gbs = None
    if not a.lean:
        copy_gbs, read_gbs = probe_bandwidth(torch, kvq, dev, 1 << 30)

    cpu = None
    if not a.no_cpu_baseline:
        import oracle
        ora = oracle.lib()
        oc = oracle.OracleCache(w.dtype, w.B, w.Hq, w.Hkv, w.boost, n_pages0 + 1)
        oc.quantize_pages(K[:, :, :bulk * PAGE], V[:, :, :bulk * PAGE])
        for t in range(n_win):
            oc.append(K[:, :, bulk * PAGE + t], V[:, :, bulk * PAGE + t])
        q0 = gen.query(w, step=0)
        # repeated full decode-attention calls until ~10 s of CPU work
        tc = time.time()
        calls = 0
        while calls < 1000 and (calls == 0 or time.time() - tc < 10.0):
            oc.attention(q0)
            calls += 1
        dt = time.time() - tc
        b = attention_bytes(w, pb, oc.n_pages, oc.n_res) * calls
        cpu = {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": ora.num_threads(),
               "kind": "oracle",
               "sample": (f"{calls} full decode-attention calls ({w.B * w.Hkv} (sequence, KV head) "
                          f"units, {oc.n_pages} pages + {oc.n_res} window tokens each, fp64) "
                          f"in {dt:.1f} s")}

    traffic = pmc_traffic("decode_split_kernel", w.name)
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_name(gen, w), "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": 128, "ctx": w.ctx, "boost_channels": w.boost,
                   "key_group": 32, "value_group": 32, "window": 128,
                   "storage": f"2-bit K/V pages + {dtype_name(gen, w)} window",
                   "accumulate": "f32", "layers_rotated": layers, "page_splits": splits,
                   "step": "append + attention, " + ("two calls" if a.unfused else "fused")},
        "tokens_per_s": round(w.B / (ms_step / 1e3), 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "attention_gbs": round(attn_gbs, 2),
        "flushes": n_flush,
        "step_us": step_dist,
        "graph_step_us": round(graph_us, 2) if graph_us else None,
        "graph_all_layers_step_us": round(graph_model_us, 2) if graph_model_us else None,
        "copy_gbs": round(copy_gbs, 1) if copy_gbs else None,
        "pct_copy_bw": round(100.0 * achieved / copy_gbs, 2) if copy_gbs else None,
        "read_gbs": round(read_gbs, 1) if read_gbs else None,
        "pct_read_bw": round(100.0 * achieved / read_gbs, 2) if read_gbs else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "kernel_us": round(kern_avg_s * 1e6, 2), "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def stream_main(a, w, torch, gen, kvq):
    """The long-context streaming workload: bulk quantization of the prefill
    (timed once, after an untimed pass on a scratch cache), then its decode
    steps, each an append plus a decode attention on every one of L layer
    replicas in turn (L sized to defeat the Infinity Cache), timed per step."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    bulk = w.prefill_pages
    print(f"[bench] workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} prefill {bulk} pages, "
          f"{w.decode_steps} decode steps", file=sys.stderr, flush=True)
    K, V = gen.prefill_kv(w, ntok=bulk * PAGE)
    Kd, Vd = to_dev(K), to_dev(V)
    if a.no_cpu_baseline:
        del K, V
    cfg = kvq.config(w.B, w.Hq, w.Hkv, w.boost, w.max_pages, w.dtype)
    scratch = kvq.Cache(cfg, device=dev)
    base = kvq.Cache(cfg, device=dev)
    rel = None
    if a.query_aware:
        rel = torch.empty(w.B, w.Hkv, 128, dtype=torch.float32, device=dev)
        kvq.kvq_query_relevance(w.dtype, w.B, w.Hq, w.Hkv, to_dev(gen.query(w, step=1)), rel)
        scratch.set_relevance(rel)
        base.set_relevance(rel)
    scratch.quantize_page(Kd, Vd, bulk)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    base.quantize_page(Kd, Vd, bulk)
    e1.record()
    torch.cuda.synchronize()
    q_ms = e0.elapsed_time(e1)
    pb = base.page_bytes
    units = w.B * w.Hkv
    q_in = units * bulk * PAGE * 128 * 2 * 2
    q_out = units * bulk * pb
    del scratch, Kd, Vd
    layers = max(2, math.ceil(a.rotate_bytes / base.nbytes))
    print(f"[bench] {layers} layer replicas (replica bytes {base.nbytes})", file=sys.stderr,
          flush=True)
    caches = [base]
    for _ in range(layers - 1):
        c = kvq.Cache(cfg, device=dev)
        c.mem.copy_(base.mem)
        kvq.kvq_set_state(c.handle, bulk, 0)
        if rel is not None:
            c.set_relevance(rel)
        caches.append(c)
    if a.splits:
        for c in caches:
            kvq.kvq_set_decode_splits(c.handle, a.splits)
    qs, kts, vts = [], [], []
    for s in range(1, w.decode_steps + 1):
        qs.append(to_dev(gen.query(w, step=s)))
        kt, vt = gen.step_kv(w, s)
        kts.append(to_dev(kt))
        vts.append(to_dev(vt))
    out = torch.empty(w.B, w.Hq, 128, dtype=torch.float32, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(w.decode_steps)]
    # the split kernel's own dispatch timestamps on layer 0 of every step
    hev = HipEvents(w.decode_steps, a.event_fence)
    torch.cuda.synchronize()
    flush_step = None
    bytes_steps, split_bytes = [], []
    # launch arguments as plain integers, resolved once (the host then issues
    # a layer step in little more than the C call itself)
    sp = torch.cuda.current_stream().cuda_stream
    kp = [t.data_ptr() for t in kts]
    vp = [t.data_ptr() for t in vts]
    qp = [t.data_ptr() for t in qs]
    op = out.data_ptr()
    hw = [(c.handle, c.ws.data_ptr(), c.ws_bytes) for c in caches]
    # one untimed attention call (it changes no state) loads the kernels the
    # steps launch, so the first timed step pays no one-time set-up
    kvq.kvq_decode_attention(hw[0][0], qp[0], op, hw[0][1], hw[0][2], sp)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(w.decode_steps):
        evs[i][0].record()
        for li, (h, wsp, wsb) in enumerate(hw):
            if li == 0:
                kvq.kvq_set_kernel_events(h, *hev.pair(i))
            if a.unfused:
                flushed = kvq.kvq_append_token(h, kp[i], vp[i], sp)
                kvq.kvq_decode_attention(h, qp[i], op, wsp, wsb, sp)
            else:
                flushed = kvq.kvq_append_decode(h, kp[i], vp[i], qp[i], op, wsp, wsb, sp)
            if li == 0:
                kvq.kvq_set_kernel_events(h, None, None)
        evs[i][1].record()
        if flushed:
            flush_step = i + 1
        n_pages, n_res = caches[0].state
        ab = attention_bytes(w, pb, n_pages, n_res)
        bytes_steps.append(ab + append_bytes(w, pb, flushed))
        split_bytes.append(ab - w.B * w.Hq * 128 * 4)  # pages + window + query
    end.record()
    torch.cuda.synchronize()
    step_ms = np.array([x.elapsed_time(y) for x, y in evs]) / layers  # per layer step
    total_ms = start.elapsed_time(end)
    value = float(np.sum(bytes_steps)) * layers / (total_ms / 1e3) / 1e9
    kern_s = np.array([hev.elapsed_ms(i) for i in range(w.decode_steps)]) / 1e3
    achieved = float(np.mean(np.array(split_bytes) / kern_s)) / 1e9
    print(f"[bench] {w.decode_steps} steps x {layers} layers in {total_ms:.3f} ms; split kernel "
          f"{kern_s.mean() * 1e6:.1f} us mean ({achieved:.0f} GB/s)", file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = stream_cpu_baseline(w, gen, K, V, pb)
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": w.decode_steps, "warmup": 0,
        "ms_per_step": round(total_ms / w.decode_steps / layers, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_name(gen, w), "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": 128, "ctx": bulk * PAGE, "decode_steps": w.decode_steps,
                   "boost_channels": w.boost, "layers_rotated": layers,
                   "channel_ranking": "query-aware" if a.query_aware else "magnitude",
                   "step": "append + attention, " + ("two calls" if a.unfused else "fused")},
        "tokens_per_s": round(w.B / (total_ms / w.decode_steps / layers / 1e3), 1),
        "step_us": {"p10": round(float(np.percentile(step_ms, 10)) * 1e3, 2),
                    "median": round(float(np.median(step_ms)) * 1e3, 2),
                    "p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2),
                    "first": round(float(step_ms[0]) * 1e3, 2),
                    "max": round(float(step_ms.max()) * 1e3, 2),
                    "flush_step": flush_step,
                    "flush_step_us": round(float(step_ms[flush_step - 1]) * 1e3, 2)
                    if flush_step else None},
        "prefill_quantize": {"pages": units * bulk, "ms": round(q_ms, 3),
                             "gbs": round((q_in + q_out) / (q_ms / 1e3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "kernel_us": round(float(kern_s.mean()) * 1e6, 2),
                     "traffic": pmc_traffic("decode_split_kernel", w.name)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def stream_cpu_baseline(w, gen, K, V, pb):
    """The oracle on the long-context stream: its own quantization of the
    prefill pages (timed, reported beside), then the decode steps' appends
    with decode attention timed at steps 1, 128, 129 (after the flush) and
    256, in fp64 on the host cores."""
    import oracle
    ora = oracle.lib()
    oc = oracle.OracleCache(w.dtype, w.B, w.Hq, w.Hkv, w.boost, w.max_pages)
    tq = time.time()
    oc.quantize_pages(K, V)
    tq = time.time() - tq
    units = w.B * w.Hkv
    q_bytes = units * w.prefill_pages * (PAGE * 128 * 2 * 2 + pb)
    at_bytes, at_s = 0, 0.0
    for s in range(1, w.decode_steps + 1):
        kt, vt = gen.step_kv(w, s)
        oc.append(kt, vt)
        if s in (1, 128, 129, 256):
            q = gen.query(w, step=s)
            tc = time.time()
            oc.attention(q)
            at_s += time.time() - tc
            at_bytes += attention_bytes(w, pb, oc.n_pages, oc.n_res)
    return {"value": round(at_bytes / at_s / 1e9, 4), "unit": "GB/s", "cores": ora.num_threads(),
            "kind": "oracle",
            "sample": (f"fp64 decode attention at steps 1, 128, 129, 256 ({units} units of "
                       f"{w.prefill_pages}-{w.prefill_pages + 1} pages + window) in {at_s:.1f} s"),
            "quantize": {"gbs": round(q_bytes / tq / 1e9, 4),
                         "sample": f"{units * w.prefill_pages} prefill pages in {tq:.1f} s"}}


def prefill_flops(T, Hq):
    """Algorithmic flops of one prefill selection: causal Q K^T and P V of the
    attention (2 T^2 / 2 Hq D flops each) and the Q K^T the cumulative scores
    recompute (two-stage selective flash-attention, MiniKV summary)."""
    return 3.0 * T * T * Hq * 128


PREFILL_CAL_BYTES = 256 << 20


def prefill_fwd_flops(T, Hq):
    """Algorithmic flops of the causal attention kernel: Q K^T and P V over
    the T (T + 1) / 2 causal pairs of every query head, 2 flops per
    multiply-add, 128 channels."""
    return 2 * 2 * (T * (T + 1) // 2) * Hq * 128


def prefill_main(a, w, torch, gen, kvq):
    """Prefill of one sequence with cumulative attention scores and
    heavy-hitter + recent selection (kvq_prefill_select: attention output,
    scores, kept positions and the gathered kept rows), timed per call."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    T = a.tokens if a.tokens > 0 else w.ctx
    heavy = recent = int(w.select * T)
    print(f"[bench] workload {w.name}: T={T} Hq={w.Hq} Hkv={w.Hkv} heavy={heavy} recent={recent}",
          file=sys.stderr, flush=True)
    q = gen.prefill_q(w, T)
    K, V = gen.prefill_kv(w, ntok=T)
    qd, kd, vd = to_dev(q), to_dev(K[0]), to_dev(V[0])
    rec = min(recent, T)
    nk = min(heavy, T - rec) + rec
    out = torch.empty(w.Hq, T, 128, dtype=torch.float32, device=dev)
    score = torch.empty(w.Hkv, T, dtype=torch.float32, device=dev)
    keep = torch.empty(w.Hkv, nk, dtype=torch.int32, device=dev)
    k_sel = torch.empty(w.Hkv, nk, 128, dtype=torch.int16, device=dev)
    v_sel = torch.empty_like(k_sel)
    wsb = kvq.kvq_prefill_workspace_bytes(T, w.Hq, w.Hkv)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    # one device copy of known size: the reference that scales HBM counters
    cal = torch.empty(PREFILL_CAL_BYTES, dtype=torch.uint8, device=dev)
    torch.empty_like(cal).copy_(cal)
    print(f"[bench] calibration copy of {PREFILL_CAL_BYTES} bytes", file=sys.stderr, flush=True)
    del cal

    def call():
        kvq.kvq_prefill_select(w.dtype, T, w.Hq, w.Hkv, 0.0, qd, kd, vd, heavy, recent, out,
                               score, keep, k_sel, v_sel, ws, wsb)

    steps = max(1, min(a.steps, 50))
    warm = max(1, min(a.warmup, 5))
    for _ in range(warm):
        call()
    # HIP events around the attention kernel on every 4th timed call
    timed = [i for i in range(steps) if a.event_every > 0 and i % a.event_every == 0]
    hev = HipEvents(len(timed), a.event_fence)
    ev_of = {i: hev.pair(j) for j, i in enumerate(timed)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        ev = ev_of.get(i)
        if ev is not None:
            kvq.kvq_prefill_set_kernel_events(ev[0], ev[1])
        call()
        if ev is not None:
            kvq.kvq_prefill_set_kernel_events(None, None)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = prefill_flops(T, w.Hq)
    tf = fl / (ms / 1e3) / 1e12
    kus = [hev.elapsed_ms(j) * 1e3 for j in range(len(timed))]
    k_us = sum(kus) / len(kus) if kus else None
    k_tf = prefill_fwd_flops(T, w.Hq) / (k_us / 1e6) / 1e12 if kus else None
    print(f"[bench] {steps} calls, {ms * 1e3:.1f} us per call, {tf:.1f} TFLOP/s algorithmic; "
          f"attention kernel {k_us:.1f} us, {k_tf:.1f} TFLOP/s" if kus else
          f"[bench] {steps} calls, {ms * 1e3:.1f} us per call, {tf:.1f} TFLOP/s algorithmic",
          file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu_baseline:
        import oracle
        ora = oracle.lib()
        T0 = min(T, 8192)  # the oracle on the first T0 positions (~10-15 s of host work)
        tc = time.time()
        ora.prefill_attention(w.dtype, q[:, :T0], K[0][:, :T0], V[0][:, :T0], 1.0 / np.sqrt(128))
        dt = time.time() - tc
        cpu = {"value": round(prefill_flops(T0, w.Hq) / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": min(ora.num_threads(), w.Hkv), "kind": "oracle",
               "sample": f"fp64 prefill attention + cumulative scores of the first {T0} positions "
                         f"({w.Hq} query heads) in {dt:.1f} s"}
    rec_ = {
        "metric": "prefill attention + cumulative scores + heavy-hitter/recent selection, "
                  "algorithmic TFLOP/s (one sequence)",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == gen.BF16 else "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": 128, "heavy": heavy, "recent": recent, "kept": nk},
        "roofline": {"bound": "mfma", "kernel": "prefill_fwd_kernel",
                     "achieved": round(k_tf, 2) if k_tf else None, "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(k_tf / 2500.0, 4) if k_tf else None,
                     "kernel_us": round(k_us, 2) if k_us else None,
                     "traffic": pmc_traffic("prefill_fwd_kernel", w.name)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec_), flush=True)


def pool_cpu_baseline(w, gen, lengths, pb):
    """The oracle's fp64 decode attention over the batch's sequences, one at a
    time (each with its own page count and window, the oracle's own pages),
    until ~10 s of attention work."""
    import oracle
    ora = oracle.lib()
    at_bytes, at_s, done = 0, 0.0, 0
    q_all = gen.query(w, step=0)
    for b, n in enumerate(lengths):
        K = np.empty((1, w.Hkv, n, 128), np.uint16)
        V = np.empty_like(K)
        for h in range(w.Hkv):
            K[0, h], V[0, h] = gen.unit_kv(w, b, h, n)
        n_pages = n // PAGE
        oc = oracle.OracleCache(w.dtype, 1, w.Hq, w.Hkv, w.boost, max(n_pages, 1))
        if n_pages:
            oc.quantize_pages(K[:, :, :n_pages * PAGE], V[:, :, :n_pages * PAGE])
        for t in range(n_pages * PAGE, n):
            oc.append(K[:, :, t], V[:, :, t])
        tc = time.time()
        oc.attention(q_all[b:b + 1])
        at_s += time.time() - tc
        at_bytes += w.Hkv * (oc.n_pages * pb + oc.n_res * 2 * 128 * 2) + w.Hq * 128 * (2 + 4)
        done += 1
        if at_s > 10.0:
            break
    return {"value": round(at_bytes / at_s / 1e9, 4), "unit": "GB/s", "cores": ora.num_threads(),
            "kind": "oracle",
            "sample": (f"fp64 decode attention of {done} of the {len(lengths)} sequences "
                       f"({sum(lengths[:done])} tokens) in {at_s:.1f} s")}


def pool_main(a, w, torch, gen, kvq):
    """A variable-length batch in the block pool: every sequence prefilled
    with its own length (pages in pool blocks, the tail in its window), then
    decode steps (append + attention of every sequence, fused) rotating over
    pool replicas sized to defeat the Infinity Cache."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    t0 = time.time()
    lengths = [int(x) for x in gen.seq_lengths(w)]
    print(f"[bench] workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} k={w.boost} lengths "
          f"{min(lengths)}..{max(lengths)} (mean {np.mean(lengths):.0f})", file=sys.stderr,
          flush=True)
    steps_total = a.warmup + a.steps
    cfg = kvq.config(w.B, w.Hq, w.Hkv, w.boost, w.max_pages + steps_total // PAGE + 2, w.dtype)
    n_blocks = sum(n // PAGE for n in lengths) + w.B * (steps_total // PAGE + 2)
    kv = []
    for b, n in enumerate(lengths):
        K = np.empty((w.Hkv, n, 128), np.uint16)
        V = np.empty_like(K)
        for h in range(w.Hkv):
            K[h], V[h] = gen.unit_kv(w, b, h, n)
        kv.append((to_dev(K), to_dev(V)))

    def make_pool():
        p = kvq.Pool(cfg, n_blocks, device=dev)
        for b in range(w.B):  # reverse order: blocks of a sequence are not adjacent in id order
            s = w.B - 1 - b
            p.prefill(s, *kv[s])
        return p

    base = make_pool()
    torch.cuda.synchronize()
    layers = max(2, math.ceil(a.rotate_bytes / base.nbytes))
    pools = [base] + [make_pool() for _ in range(layers - 1)]
    del kv
    # one device copy of known size: the reference that scales HBM traffic
    # counters of a profiled run of this benchmark
    calib = torch.empty_like(base.mem)
    calib.copy_(base.mem)
    del calib
    qs, kts, vts = [], [], []
    for s in range(steps_total):
        qs.append(to_dev(gen.query(w, step=s)))
        kt, vt = gen.step_kv(w, s)
        kts.append(to_dev(kt))
        vts.append(to_dev(vt))
    out = torch.empty(w.B, w.Hq, 128, dtype=torch.float32, device=dev)
    timed = [i for i in range(a.steps) if a.event_every > 0 and i % a.event_every == 0]
    hev = HipEvents(len(timed), a.event_fence)
    ev_of = {i: hev.pair(j) for j, i in enumerate(timed)}
    torch.cuda.synchronize()
    pb = base.page_bytes
    print(f"[bench] setup {time.time() - t0:.1f}s; {layers} pool replicas of "
          f"{base.nbytes / 1e6:.1f} MB (replica bytes {base.nbytes})", file=sys.stderr, flush=True)

    def seq_states(p):
        return [p.seq(b) for b in range(w.B)]

    def step_bytes(states, flushes):
        """Pages and window tokens of every live sequence, q, output; the
        appends, and per flush a window read and a page write."""
        att = sum(w.Hkv * (n_pages * pb + n_res * 2 * 128 * 2)
                  for live, n_pages, n_res in states if live)
        att += w.B * w.Hq * 128 * 2 + w.B * w.Hq * 128 * 4
        app = w.B * w.Hkv * 2 * 128 * 2 * 2 + flushes * w.Hkv * (128 * 128 * 2 * 2 + pb)
        return att, app

    for s in range(a.warmup):
        pools[s % layers].append_decode(kts[s], vts[s], qs[s], out)
    torch.cuda.synchronize()
    # launch arguments as plain integers, resolved once; the slots' counters
    # tracked here (a full window is flushed before its token goes in) and
    # checked against the library's after the timed steps
    sp = torch.cuda.current_stream().cuda_stream
    kp = [t.data_ptr() for t in kts]
    vp = [t.data_ptr() for t in vts]
    qp = [t.data_ptr() for t in qs]
    op = out.data_ptr()
    hw = [(p.handle, p.ws.data_ptr(), p.ws_bytes) for p in pools]
    tracked = [[list(x) for x in seq_states(p)] for p in pools]

    def track(states):
        nf = 0
        for e in states:
            if e[0]:
                if e[2] == PAGE:
                    e[1], e[2], nf = e[1] + 1, 0, nf + 1
                e[2] += 1
        return nf

    total_bytes, split_bytes, n_flush = 0, [], 0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(a.steps):
        s = a.warmup + i
        h, wsp, wsb = hw[s % layers]
        ev = ev_of.get(i)
        if ev is not None:
            kvq.kvq_pool_set_kernel_events(h, ev[0], ev[1])
        nf = kvq.kvq_pool_append_decode(h, kp[s], vp[s], qp[s], op, wsp, wsb, sp)
        if ev is not None:
            kvq.kvq_pool_set_kernel_events(h, None, None)
        st = tracked[s % layers]
        assert track(st) == nf
        att, app = step_bytes(st, nf)
        total_bytes += att + app
        n_flush += nf
        if ev is not None:
            split_bytes.append(att - w.B * w.Hq * 128 * 4)
    end.record()
    torch.cuda.synchronize()
    assert all([tuple(e) for e in tracked[li]] == seq_states(p) for li, p in enumerate(pools))
    ms = start.elapsed_time(end)
    ms_step = ms / a.steps
    kern_ms = np.array([hev.elapsed_ms(j) for j in range(len(timed))])
    kern_avg_s = float(kern_ms.mean()) / 1e3
    achieved = float(np.mean(split_bytes)) / kern_avg_s / 1e9
    value = total_bytes / (ms / 1e3) / 1e9
    print(f"[bench] {a.steps} steps in {ms:.3f} ms ({ms_step * 1e3:.1f} us/step, pool split "
          f"kernel avg {kern_avg_s * 1e6:.1f} us over {len(timed)} launches, {n_flush} flushes)",
          file=sys.stderr, flush=True)
    rec = {
        "metric": METRIC + " (variable-length batch, block pool)", "value": round(value, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype_name(gen, w), "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": 128, "lengths": lengths, "boost_channels": w.boost,
                   "layers_rotated": layers, "step": "append + attention, fused (pool)"},
        "tokens_per_s": round(w.B / (ms_step / 1e3), 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": pmc_traffic("pool_split_kernel", w.name)},
        "cpu_baseline": None if a.no_cpu_baseline else pool_cpu_baseline(w, gen, lengths, pb),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
