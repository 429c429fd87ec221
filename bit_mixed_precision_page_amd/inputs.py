"""Seeded synthetic decode workloads (inputs only; none of the method's arithmetic).

Every array is drawn from numpy's PCG64 with a seed derived from the workload,
a role and the (sequence, KV head) unit, so any unit can be regenerated alone.
Values are drawn in float32 and rounded once (round-to-nearest-even, by numpy
for fp16 and by torch for bf16) to the storage dtype; they travel as uint16
bit patterns.  fp16 draws are clamped to +-60000 first.

Key distributions model the activation statistics the pages describe: Keys
carry per-channel outliers (MiniKV summary, "proposed method"; KIVI explainer,
section 3), Values and queries are plain Gaussians.  Outlier channel sets are a
property of the KV head, shared by every sequence and token.
"""
from dataclasses import dataclass

import numpy as np

F16, BF16 = 0, 1
HEAD_DIM = 128
PAGE = 128
RESIDUAL = 128

(ROLE_CHANNELS, ROLE_K, ROLE_V, ROLE_Q, ROLE_STEP_K, ROLE_STEP_V, ROLE_STEP_Q,
 ROLE_LENGTHS, ROLE_PREFILL_Q) = range(9)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # seed id
    B: int
    Hq: int
    Hkv: int
    ctx: int            # tokens in the cache when attention is measured
    boost: int          # boosted Key channels per page (of 128)
    dtype: int          # F16 or BF16
    k_dist: str         # "outlier", "logscale", "student_t"
    outliers: int = 0   # outlier channels per KV head ("outlier")
    outlier_gain: float = 1.0
    decode_steps: int = 0  # streaming steps after the prefill
    ctx_spread: int = 0    # variable-length batch: lengths uniform in ctx +- ctx_spread
    select: float = 0.0    # prefill with token selection: heavy and recent share of ctx each

    @property
    def seed(self):
        return 20260000 + self.wid

    @property
    def g(self):
        return self.Hq // self.Hkv

    @property
    def prefill_pages(self):
        """Pages written by bulk quantization before the measured state."""
        if self.decode_steps:
            return self.ctx // PAGE
        return self.ctx // PAGE - 1

    @property
    def prefill_residual(self):
        """Tokens appended one by one after the bulk pages."""
        return 0 if self.decode_steps else RESIDUAL

    @property
    def max_pages(self):
        return (self.ctx + self.ctx_spread + self.decode_steps) // PAGE + 1


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 1, 1, 4, 1, 1024, 16, F16, "outlier", 8, 10.0),
        Workload("llama3_8b_decode", 2, 16, 32, 8, 8192, 16, BF16, "outlier", 6, 8.0),
        Workload("qwen3_8b_long", 3, 8, 32, 8, 32768, 32, BF16, "logscale"),
        Workload("llama70b_large_batch", 4, 128, 64, 8, 4096, 16, BF16, "outlier", 6, 8.0),
        Workload("long_prefill_decode", 5, 1, 32, 8, 131072, 16, BF16, "student_t",
                 decode_steps=256),
        Workload("llama3_8b_varlen", 6, 16, 32, 8, 8192, 16, BF16, "outlier", 6, 8.0,
                 ctx_spread=7168),
        Workload("llama3_8b_prefill_select", 7, 1, 32, 8, 8192, 16, BF16, "outlier", 6, 8.0,
                 select=0.25),
    ]
}


def rng(seed, role, *unit):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, role, *unit])))


def to_bits(x, dtype):
    """float32 array -> uint16 bit patterns of the storage dtype (one RNE step)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == F16:
        return np.clip(x, -60000.0, 60000.0).astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def from_bits(bits, dtype):
    """uint16 bit patterns -> float32 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def channel_gain(w, h):
    """Per-channel standard deviation of Keys for KV head h, shape [128]."""
    r = rng(w.seed, ROLE_CHANNELS, h)
    gain = np.ones(HEAD_DIM, np.float32)
    if w.k_dist == "outlier":
        ch = r.choice(HEAD_DIM, size=w.outliers, replace=False)
        gain[ch] = w.outlier_gain
    elif w.k_dist == "logscale":
        gain = np.exp(r.uniform(np.log(0.5), np.log(16.0), HEAD_DIM)).astype(np.float32)
    return gain


def _keys(w, r, shape, gain):
    if w.k_dist == "student_t":
        return r.standard_t(3, size=shape).astype(np.float32)
    return r.standard_normal(shape, dtype=np.float32) * gain


def unit_kv(w, b, h, ntok=None):
    """Prefill K, V of one (sequence, KV head): two [ntok][128] uint16 arrays."""
    ntok = w.ctx if ntok is None else ntok
    gain = channel_gain(w, h)
    K = _keys(w, rng(w.seed, ROLE_K, b, h), (ntok, HEAD_DIM), gain)
    V = rng(w.seed, ROLE_V, b, h).standard_normal((ntok, HEAD_DIM), dtype=np.float32)
    return to_bits(K, w.dtype), to_bits(V, w.dtype)


def prefill_kv(w, ntok=None):
    """K, V [B][Hkv][ntok][128] uint16 for the whole batch."""
    ntok = w.ctx if ntok is None else ntok
    K = np.empty((w.B, w.Hkv, ntok, HEAD_DIM), np.uint16)
    V = np.empty_like(K)
    for b in range(w.B):
        for h in range(w.Hkv):
            K[b, h], V[b, h] = unit_kv(w, b, h, ntok)
    return K, V


def seq_lengths(w):
    """Tokens per sequence [B] (int): uniform in [ctx - ctx_spread, ctx + ctx_spread]."""
    if not w.ctx_spread:
        return np.full(w.B, w.ctx, np.int64)
    r = rng(w.seed, ROLE_LENGTHS)
    return r.integers(w.ctx - w.ctx_spread, w.ctx + w.ctx_spread + 1, size=w.B)


def prefill_q(w, T, b=0):
    """Prefill queries of sequence b: [Hq][T][128] uint16, N(0, 1)."""
    r = rng(w.seed, ROLE_PREFILL_Q, b)
    return to_bits(r.standard_normal((w.Hq, T, HEAD_DIM), dtype=np.float32), w.dtype)


def query(w, step=None):
    """Q [B][Hq][128] uint16 (step=None: the measured query)."""
    r = rng(w.seed, ROLE_Q) if step is None else rng(w.seed, ROLE_STEP_Q, step)
    return to_bits(r.standard_normal((w.B, w.Hq, HEAD_DIM), dtype=np.float32), w.dtype)


def step_kv(w, step):
    """K, V [B][Hkv][128] uint16 of one streamed decode token."""
    K = np.empty((w.B, w.Hkv, HEAD_DIM), np.float32)
    for h in range(w.Hkv):
        K[:, h] = _keys(w, rng(w.seed, ROLE_STEP_K, step, h), (w.B, HEAD_DIM),
                        channel_gain(w, h))
    V = rng(w.seed, ROLE_STEP_V, step).standard_normal((w.B, w.Hkv, HEAD_DIM),
                                                      dtype=np.float32)
    return to_bits(K, w.dtype), to_bits(V, w.dtype)
