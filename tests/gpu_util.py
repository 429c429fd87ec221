"""Helpers for GPU parity tests: the same seeded inputs go to the HIP path
(through the C ABI) and to the CPU oracle; nothing flows from one to the other."""
import numpy as np
import torch

import oracle
from bit_mixed_precision_page_amd import inputs as gen

P = 128
GUARD = 1 << 16  # canary bytes before and after every guarded device buffer


class Guards:
    """Device buffers with canary bands: each allocation is the middle of a
    larger tensor whose first and last GUARD bytes hold a seeded pattern.
    `check()` asserts every band is unchanged (a kernel that writes past its
    buffer, in either direction, changes one) and forgets the buffers."""

    def __init__(self):
        self.items = []
        self.n = 0

    def alloc(self, nbytes, device="cuda"):
        buf = torch.empty(nbytes + 2 * GUARD, dtype=torch.uint8, device=device)
        g = torch.Generator().manual_seed(1000 + self.n)
        self.n += 1
        pat = torch.randint(0, 256, (2, GUARD), dtype=torch.uint8, generator=g)
        buf[:GUARD].copy_(pat[0])
        buf[GUARD + nbytes:].copy_(pat[1])
        self.items.append((buf, nbytes, pat))
        return buf[GUARD:GUARD + nbytes]

    def out(self, *shape, dtype=torch.float32):
        """A guarded output tensor."""
        n = int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size()
        return self.alloc(n).view(dtype).view(*shape)

    def check(self):
        torch.cuda.synchronize()
        items, self.items = self.items, []
        for i, (buf, nbytes, pat) in enumerate(items):
            lo = buf[:GUARD].cpu()
            hi = buf[GUARD + nbytes:].cpu()
            assert torch.equal(lo, pat[0]), f"guard band before buffer {i} ({nbytes} B) overwritten"
            assert torch.equal(hi, pat[1]), f"guard band after buffer {i} ({nbytes} B) overwritten"
        return len(items)


GUARDS = Guards()


def guarded_cache(cfg):
    from bit_mixed_precision_page_amd import kvq
    return kvq.Cache(cfg, alloc=GUARDS.alloc)


def guarded_pool(cfg, n_blocks):
    from bit_mixed_precision_page_amd import kvq
    return kvq.Pool(cfg, n_blocks, alloc=GUARDS.alloc)


def assert_plan_ok(obj, mode=0):
    """The host-side extent check of the next decode launch passes."""
    rc, msg = obj.check_plan(mode)
    assert rc == 0, f"decode plan check: {msg}"


def dev(bits):
    """uint16 bit patterns -> contiguous int16 CUDA tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    return t.cpu().numpy()


def kv_for(w, B, ntok):
    K = np.empty((B, w.Hkv, ntok, 128), np.uint16)
    V = np.empty_like(K)
    for b in range(B):
        for h in range(w.Hkv):
            K[b, h], V[b, h] = gen.unit_kv(w, b, h, ntok)
    return K, V


class Pair:
    """A GPU cache and its oracle model, fed the same tokens."""

    def __init__(self, w, B=None, bulk_pages=None, window=None, boost=None, Hq=None, Hkv=None,
                 max_pages=None, with_oracle=True, scale=0.0):
        from bit_mixed_precision_page_amd import kvq
        self.kvq = kvq
        self.w = w
        self.B = w.B if B is None else B
        self.Hkv = w.Hkv if Hkv is None else Hkv
        self.Hq = w.Hq if Hq is None else Hq
        self.k = w.boost if boost is None else boost
        self.bulk = w.prefill_pages if bulk_pages is None else bulk_pages
        self.window = w.prefill_residual if window is None else window
        self.max_pages = max_pages or (self.bulk + self.window // P + 2)
        self.cfg = kvq.config(self.B, self.Hq, self.Hkv, self.k, self.max_pages, w.dtype,
                              softmax_scale=scale)
        self.gpu = guarded_cache(self.cfg)
        self.ora = (oracle.OracleCache(w.dtype, self.B, self.Hq, self.Hkv, self.k,
                                       self.max_pages, scale=scale)
                    if with_oracle else None)
        wk = w if Hkv is None else _with_hkv(w, self.Hkv)
        T = self.bulk * P + self.window
        self.K, self.V = kv_for(wk, self.B, T)
        if self.bulk:
            Kb = np.ascontiguousarray(self.K[:, :, :self.bulk * P])
            Vb = np.ascontiguousarray(self.V[:, :, :self.bulk * P])
            self.gpu.quantize_page(dev(Kb), dev(Vb), self.bulk)
            if self.ora is not None:
                self.ora.quantize_pages(Kb, Vb)
        self.flushes = []
        for t in range(self.window):
            self.append(self.K[:, :, self.bulk * P + t], self.V[:, :, self.bulk * P + t])

    def append(self, k_t, v_t):
        assert_plan_ok(self.gpu, mode=1)
        f = self.gpu.append_token(dev(k_t), dev(v_t))
        if self.ora is not None:
            fo = self.ora.append(k_t, v_t)
            assert f == fo
        self.flushes.append(f)
        return f

    def query(self, step=None):
        r = np.random.default_rng(1000 + (0 if step is None else step))
        q = gen.to_bits(r.standard_normal((self.B, self.Hq, 128), dtype=np.float32),
                        self.w.dtype)
        return q

    def attention(self, q_bits, splits=0):
        out = GUARDS.out(self.B, self.Hq, 128)
        self.kvq.kvq_set_decode_splits(self.gpu.handle, splits)
        assert_plan_ok(self.gpu)
        self.gpu.decode_attention(dev(q_bits), out)
        torch.cuda.synchronize()
        return host(out)

    def pages(self):
        torch.cuda.synchronize()
        return host(self.gpu.pages_view())

    def windows(self):
        torch.cuda.synchronize()
        k, v = self.gpu.window_view()
        return host(k).view(np.uint16), host(v).view(np.uint16)


def _with_hkv(w, Hkv):
    import dataclasses
    return dataclasses.replace(w, Hkv=Hkv, Hq=Hkv * w.g)


def first_page_mismatch(a, b):
    bad = np.argwhere((a != b).any(axis=-1))
    if len(bad) == 0:
        return None
    b_, h, p = bad[0]
    byte = int(np.flatnonzero(a[b_, h, p] != b[b_, h, p])[0])
    return f"unit ({b_},{h}) page {p} first byte {byte}: {a[b_, h, p, byte]} vs {b[b_, h, p, byte]}"
