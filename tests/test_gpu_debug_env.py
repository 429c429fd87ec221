"""The library's environment switches, in a child process of their own (they
are read once per process): KVQ_TRACE=1 prints one line per call, and
KVQ_CHECK=1 walks every decode launch (dense cache and block pool) before it
runs without changing what the calls compute."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import torch
from bit_mixed_precision_page_amd import kvq
torch.manual_seed(3)
B, Hq, Hkv = 2, 8, 2
c = kvq.Cache(kvq.config(B, Hq, Hkv, 16, 4, kvq.KVQ_BF16))
k = torch.randn(B, Hkv, 2 * 128, 128, device="cuda").bfloat16()
v = torch.randn(B, Hkv, 2 * 128, 128, device="cuda").bfloat16()
c.quantize_page(k, v, 2)
q = torch.randn(B, Hq, 128, device="cuda").bfloat16()
out = torch.zeros(B, Hq, 128, device="cuda")
for t in range(130):
    kt = torch.randn(B, Hkv, 128, device="cuda").bfloat16()
    vt = torch.randn(B, Hkv, 128, device="cuda").bfloat16()
    c.append_decode(kt, vt, q, out)
c.decode_attention(q, out)
pool = kvq.Pool(kvq.config(B, Hq, Hkv, 16, 4, kvq.KVQ_BF16), 16)
for s, n in ((0, 300), (1, 140)):
    pool.prefill(s, torch.randn(Hkv, n, 128, device="cuda").bfloat16(),
                 torch.randn(Hkv, n, 128, device="cuda").bfloat16())
pout = torch.zeros(B, Hq, 128, device="cuda")
for t in range(20):
    pool.append_decode(torch.randn(B, Hkv, 128, device="cuda").bfloat16(),
                       torch.randn(B, Hkv, 128, device="cuda").bfloat16(), q, pout)
pool.decode_attention(q, pout)
torch.cuda.synchronize()
print("STATE", *c.state, *pool.seq(0), *pool.seq(1), float(out.double().abs().sum()),
      float(pout.double().abs().sum()), flush=True)
"""


def _run(env_extra):
    env = dict(os.environ)
    env.pop("KVQ_CHECK", None)
    env.pop("KVQ_TRACE", None)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    print("child with", env_extra, flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    state = [ln for ln in r.stdout.splitlines() if ln.startswith("STATE")]
    assert len(state) == 1, r.stdout
    return state[0], r.stderr


def test_check_and_trace_switches():
    plain, err0 = _run({})
    assert "[kvq]" not in err0
    checked, err1 = _run({"KVQ_CHECK": "1", "KVQ_TRACE": "1"})
    # the same counters and the same outputs, bit for bit (one process each,
    # the same seeded inputs and the same launches)
    assert checked == plain
    # dense cache: two pages quantized, one flush, 2 in the window; pool: 300 + 20 tokens
    # (2 pages, 64 in the window) and 140 + 20 (1 page, 32)
    assert plain.split()[1:9] == ["3", "2", "True", "2", "64", "True", "1", "32"]
    lines = [ln for ln in err1.splitlines() if ln.startswith("[kvq]")]
    assert not any("refused" in ln for ln in lines), lines
    assert sum("kvq_quantize_page" in ln for ln in lines) == 1
    assert sum("kvq_append_decode" in ln for ln in lines) == 130
    assert sum("kvq_decode_attention" in ln for ln in lines) == 1
    assert sum("kvq_pool_append_decode" in ln for ln in lines) == 20
    assert sum("kvq_pool_decode_attention" in ln for ln in lines) == 1
