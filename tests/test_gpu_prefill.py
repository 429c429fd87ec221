"""Prefill attention with cumulative scores and token selection (kvq_prefill_select)
against the CPU oracle, through the C ABI.

Bars: attention output within max-abs 1e-3 of the oracle's fp64 causal
attention; cumulative scores within 1e-4 relative of the oracle's; the kept
positions equal the oracle's selection run on the GPU's own scores (the
decision is taken in the kernel's precision), and are a valid selection for
the oracle's scores up to that tolerance; gathered rows bit-exact.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from bit_mixed_precision_page_amd import inputs as gen
from gpu_util import dev, guarded_cache, host

import oracle

pytestmark = pytest.mark.gpu
TOL = 1e-3
STOL = 1e-4
W = gen.WORKLOADS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(w, T):
    K, V = gen.prefill_kv(w, ntok=T)
    return gen.prefill_q(w, T), K[0], V[0]


def _run(w, T, heavy, recent, scale=0.0, check_oracle_rows=None):
    from bit_mixed_precision_page_amd import kvq
    q, k, v = _inputs(w, T)
    out, score, keep, k_sel, v_sel = kvq.prefill_select(w.dtype, dev(q), dev(k), dev(v), heavy,
                                                        recent, softmax_scale=scale)
    torch.cuda.synchronize()
    return q, k, v, host(out), host(score), host(keep), host(k_sel).view(np.uint16), \
        host(v_sel).view(np.uint16)


def _late_rows(T, last=128, spread=64):
    """The last `last` query positions plus `spread` positions spread over the
    sequence: rows that see many 32-key blocks and many online-softmax
    rescale events."""
    rows = set(range(max(0, T - last), T)) | set(np.linspace(0, T - 1, spread).astype(int).tolist())
    return np.array(sorted(rows), np.int32)


def _check_rows(w, q, k, v, out_rows, rows, scale=None):
    """GPU output rows (out_rows [Hq][len(rows)][D]) against the oracle's fp64
    causal attention of the same query positions."""
    sc = 1.0 / np.sqrt(128) if scale is None else scale
    ref = oracle.lib().prefill_rows(w.dtype, q, k, v, sc, rows)
    err = np.abs(out_rows - ref).max()
    assert np.isfinite(out_rows).all()
    return err


def _check(w, T, heavy, recent, scale=0.0):
    ora = oracle.lib()
    q, k, v, out, score, keep, k_sel, v_sel = _run(w, T, heavy, recent, scale)
    sc = scale if scale > 0 else 1.0 / np.sqrt(128)
    o_ref, s_ref = ora.prefill_attention(w.dtype, q, k, v, sc)
    err = np.abs(out - o_ref).max()
    serr = (np.abs(score - s_ref) / (1.0 + np.abs(s_ref))).max()
    say(f"    T={T} Hq={w.Hq} Hkv={w.Hkv} heavy={heavy} recent={recent}: "
        f"|out - oracle| = {err:.2e}, score rel = {serr:.2e}, kept {keep.shape[1]}")
    assert np.isfinite(out).all() and np.isfinite(score).all()
    assert err <= TOL
    assert serr <= STOL
    g = w.Hq // w.Hkv
    assert np.allclose(score.sum(axis=1), g * T, rtol=1e-5)
    for h in range(w.Hkv):
        # the decision in the kernel's precision: the oracle's rule on the GPU's scores
        want = ora.select_tokens(score[h].astype(np.float64), heavy, recent)
        assert keep[h].tolist() == want.tolist(), f"KV head {h}: selection differs"
        # and a valid selection for the oracle's own scores, up to the score tolerance
        rec = min(recent, T)
        n_old = T - rec
        kept = set(keep[h].tolist())
        cand_kept = [j for j in range(n_old) if j in kept]
        cand_drop = [j for j in range(n_old) if j not in kept]
        if cand_kept and cand_drop:
            lo = s_ref[h, cand_kept].min()
            hi = s_ref[h, cand_drop].max()
            assert lo >= hi - STOL * (1.0 + hi) * 4, (h, lo, hi)
        assert all(j in kept for j in range(n_old, T))
        assert (k_sel[h] == k[h, keep[h]]).all() and (v_sel[h] == v[h, keep[h]]).all()
    return out, score, keep


@pytest.mark.parametrize("T", [1, 31, 300])
def test_prefill_bf16_gqa4(T):
    w = dataclasses.replace(W["llama3_8b_prefill_select"], Hq=8, Hkv=2)
    _check(w, T, heavy=T // 4, recent=T // 4)


def test_prefill_fp16_group_sizes():
    base = W["tiny"]
    # group sizes 8, 1, 16 (four heads per workgroup, or one), 3 (one), 6 (two)
    for Hq, Hkv, T in [(8, 1, 129), (2, 2, 70), (16, 1, 40), (6, 2, 200), (12, 2, 97)]:
        w = dataclasses.replace(base, Hq=Hq, Hkv=Hkv)
        _check(w, T, heavy=17, recent=9)


def test_prefill_selection_edges():
    w = dataclasses.replace(W["llama3_8b_prefill_select"], Hq=4, Hkv=2)
    _check(w, 100, heavy=0, recent=0)      # nothing kept
    _check(w, 100, heavy=500, recent=30)   # every candidate kept
    _check(w, 100, heavy=10, recent=400)   # the window covers everything
    _check(w, 64, heavy=64, recent=0, scale=0.2)  # explicit scale


@pytest.mark.parametrize("cap", [1, 2])
def test_prefill_forced_key_splits(cap):
    """Short sequences normally take the key-split path; with the chunk count
    capped at 1 the unsplit multi-block path (lazy rescale over many 32-key
    blocks) runs, and with 2 a two-chunk split: every output row, score and
    kept position against the oracle."""
    from bit_mixed_precision_page_amd import kvq
    w = dataclasses.replace(W["llama3_8b_prefill_select"], Hq=8, Hkv=2)
    kvq.kvq_prefill_set_max_key_splits(cap)
    try:
        for T in (300, 777):
            _check(w, T, heavy=T // 4, recent=T // 4)
    finally:
        kvq.kvq_prefill_set_max_key_splits(0)


def test_prefill_selected_rows_quantize_like_the_oracle():
    """The kept rows (two full pages here) go through kvq_quantize_page: page
    bytes bit-exact with the oracle's pages of the same rows."""
    from bit_mixed_precision_page_amd import kvq
    w = dataclasses.replace(W["llama3_8b_prefill_select"], Hq=8, Hkv=2)
    T, heavy, recent = 512, 128, 128
    q, k, v = _inputs(w, T)
    out, score, keep, k_sel, v_sel = kvq.prefill_select(w.dtype, dev(q), dev(k), dev(v), heavy,
                                                        recent)
    cfg = kvq.config(1, w.Hq, w.Hkv, w.boost, 2, w.dtype)
    cache = guarded_cache(cfg)
    cache.quantize_page(k_sel.contiguous()[None], v_sel.contiguous()[None], 2)
    torch.cuda.synchronize()
    ks = host(k_sel).view(np.uint16)[None]
    vs = host(v_sel).view(np.uint16)[None]
    ora = oracle.OracleCache(w.dtype, 1, w.Hq, w.Hkv, w.boost, 2)
    ora.quantize_pages(ks, vs)
    assert (host(cache.pages_view()) == ora.pages).all()


def test_prefill_full_size_sampled():
    """The benchmark shape (one Llama-3-8B-shaped sequence of 8192 tokens): rows
    0..383 against the oracle run on the first 384 positions (causal: those
    rows see nothing later), the last 128 rows and 64 rows spread over the
    sequence (every query head) against the oracle's rows, the last key's
    score against its single softmax probability per head, score totals, and
    the selection rule on the GPU's scores."""
    from bit_mixed_precision_page_amd import kvq
    w = W["llama3_8b_prefill_select"]
    T = w.ctx
    heavy = recent = int(w.select * T)
    q, k, v = _inputs(w, T)
    out, score, keep, k_sel, v_sel = kvq.prefill_select(w.dtype, dev(q), dev(k), dev(v), heavy,
                                                        recent)
    torch.cuda.synchronize()
    out, score, keep = host(out), host(score), host(keep)
    ora = oracle.lib()
    T0 = 384
    o_ref, _ = ora.prefill_attention(w.dtype, q[:, :T0], k[:, :T0], v[:, :T0], 1.0 / np.sqrt(128))
    err = np.abs(out[:, :T0] - o_ref).max()
    rows = _late_rows(T)
    rerr = _check_rows(w, q, k, v, out[:, rows], rows)
    say(f"    full size: {len(rows)} late and spread rows of every query head "
        f"|out - oracle| = {rerr:.2e}")
    assert rerr <= TOL
    g = w.Hq // w.Hkv
    qf = gen.from_bits(q[:, T - 1], w.dtype).astype(np.float64)
    kf = gen.from_bits(k, w.dtype).astype(np.float64)
    last = []
    for h in range(w.Hkv):
        s = qf[h * g:(h + 1) * g] @ kf[h].T / np.sqrt(128)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        last.append(p[:, T - 1].sum())
    lerr = np.abs(score[:, T - 1] - np.array(last)).max()
    say(f"    full size: rows 0..{T0 - 1} |out - oracle| = {err:.2e}, last-key score err "
        f"{lerr:.2e}, score totals {score.sum(axis=1).min():.1f}..{score.sum(axis=1).max():.1f}")
    assert err <= TOL
    assert lerr <= 1e-5
    assert np.allclose(score.sum(axis=1), g * T, rtol=1e-4)
    for h in range(w.Hkv):
        want = ora.select_tokens(score[h].astype(np.float64), heavy, recent)
        assert keep[h].tolist() == want.tolist()


def test_prefill_long_sequence_sampled():
    """A 65536-token sequence (two KV heads, eight query heads): the first 256
    rows, the last 128 rows and 64 rows spread over the sequence against the
    oracle, the last key's score against its softmax
    probabilities, the score totals, and the selection rule on the GPU scores
    (many query chunks, every tile count of the score pass past its first)."""
    from bit_mixed_precision_page_amd import kvq
    w = dataclasses.replace(W["llama3_8b_prefill_select"], Hq=8, Hkv=2, ctx=65536)
    T = w.ctx
    heavy = recent = T // 8
    q, k, v = _inputs(w, T)
    out, score, keep, k_sel, v_sel = kvq.prefill_select(w.dtype, dev(q), dev(k), dev(v), heavy,
                                                        recent)
    torch.cuda.synchronize()
    score, keep = host(score), host(keep)
    out0 = host(out[:, :256])
    rows = _late_rows(T)
    out_rows = host(out[:, torch.from_numpy(rows.astype(np.int64)).cuda()])
    del out, k_sel, v_sel
    ora = oracle.lib()
    T0 = 256
    o_ref, _ = ora.prefill_attention(w.dtype, q[:, :T0], k[:, :T0], v[:, :T0], 1.0 / np.sqrt(128))
    err = np.abs(out0 - o_ref).max()
    rerr = _check_rows(w, q, k, v, out_rows, rows)
    say(f"    T={T}: {len(rows)} late and spread rows |out - oracle| = {rerr:.2e}")
    assert rerr <= TOL
    g = w.Hq // w.Hkv
    qf = gen.from_bits(q[:, T - 1], w.dtype).astype(np.float64)
    kf = gen.from_bits(k, w.dtype).astype(np.float64)
    last = []
    for h in range(w.Hkv):
        s = qf[h * g:(h + 1) * g] @ kf[h].T / np.sqrt(128)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        last.append(p[:, T - 1].sum())
    lerr = np.abs(score[:, T - 1] - np.array(last)).max()
    say(f"    T={T}: rows 0..{T0 - 1} |out - oracle| = {err:.2e}, last-key score err {lerr:.2e}, "
        f"score totals {score.sum(axis=1).min():.1f}..{score.sum(axis=1).max():.1f}")
    assert err <= TOL
    assert lerr <= 1e-5
    assert np.allclose(score.sum(axis=1), g * T, rtol=1e-4)
    for h in range(w.Hkv):
        want = ora.select_tokens(score[h].astype(np.float64), heavy, recent)
        assert keep[h].tolist() == want.tolist()


def test_prefill_timing_hook():
    """kvq_prefill_set_kernel_events: the attention kernel's own dispatch
    timestamps land in the two events; the outputs are those of a call
    without the hook; clearing it leaves later calls untimed."""
    import ctypes
    from bit_mixed_precision_page_amd import kvq
    hip = ctypes.CDLL("libamdhip64.so")
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    w = dataclasses.replace(W["llama3_8b_prefill_select"], Hq=8, Hkv=2)
    T = 1024
    q, k, v = _inputs(w, T)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ref = kvq.prefill_select(w.dtype, qd, kd, vd, 64, 64)
    kvq.kvq_prefill_set_kernel_events(ev[0].value, ev[1].value)
    try:
        got = kvq.prefill_select(w.dtype, qd, kd, vd, 64, 64)
        torch.cuda.synchronize()
    finally:
        kvq.kvq_prefill_set_kernel_events(None, None)
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    say(f"    attention kernel {ms.value * 1e3:.1f} us")
    assert 0.0 < ms.value < 1000.0
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    for e in ev:
        hip.hipEventDestroy(e)
