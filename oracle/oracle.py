"""Python face of the CPU oracle (test infrastructure only).

Thin ctypes wrappers over ``kvq_oracle.c`` plus `OracleCache`, a host model of
one quantized KV cache: bulk page quantization, streaming append with the
flush-before-insert window, and double-precision decode attention.  Stored
values (fp16 / bf16) travel as ``uint16`` bit patterns.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module.  It never imports the product package.
"""
import ctypes
import os

import numpy as np

from . import build as _build

D = 128
P = 128
GK = 32
GV = 32
R = 128
F16, BF16 = 0, 1

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)


def _ptr(a, t):
    return a.ctypes.data_as(t)


class OracleLib:
    """ctypes handle on one build of the oracle (plant=0 is the oracle)."""

    def __init__(self, path):
        self.path = path
        L = ctypes.CDLL(path)
        L.ora_decode.restype = ctypes.c_double
        L.ora_decode.argtypes = [ctypes.c_int, ctypes.c_uint16]
        L.ora_encode.restype = ctypes.c_uint16
        L.ora_encode.argtypes = [ctypes.c_int, ctypes.c_double]
        L.ora_quantize_group.restype = None
        L.ora_quantize_group.argtypes = [ctypes.c_int, _u16p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, _u16p, _u16p, _u8p, ctypes.c_int]
        L.ora_select_channels.restype = None
        L.ora_select_channels.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          _u8p, _u8p]
        L.ora_page_bytes.restype = ctypes.c_size_t
        L.ora_page_bytes.argtypes = [ctypes.c_int]
        L.ora_page_layout.restype = None
        L.ora_page_layout.argtypes = [ctypes.c_int, _i64p]
        L.ora_vcode_bit.restype = ctypes.c_size_t
        L.ora_vcode_bit.argtypes = [ctypes.c_int, ctypes.c_int]
        L.ora_klo_bit.restype = ctypes.c_size_t
        L.ora_klo_bit.argtypes = [ctypes.c_int, ctypes.c_int]
        L.ora_khi_bit.restype = ctypes.c_size_t
        L.ora_khi_bit.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.ora_quantize_page.restype = ctypes.c_int
        L.ora_quantize_page.argtypes = [ctypes.c_int, ctypes.c_int, _u16p, _u16p, _u8p,
                                        _u8p, _u8p]
        L.ora_unpack_page.restype = ctypes.c_int
        L.ora_unpack_page.argtypes = [ctypes.c_int, ctypes.c_int, _u8p, _u8p, _u8p, _u8p,
                                      _u8p, _u16p, _u16p, _u16p, _u16p, _u8p]
        L.ora_dequantize_page.restype = ctypes.c_int
        L.ora_dequantize_page.argtypes = [ctypes.c_int, ctypes.c_int, _u8p, _f64p, _f64p]
        L.ora_attention.restype = ctypes.c_int
        L.ora_attention.argtypes = [ctypes.c_int] * 8 + [_u8p, _u16p, _u16p, _u16p,
                                                         ctypes.c_double, _f64p,
                                                         ctypes.c_int, ctypes.c_int]
        L.ora_select_channels_rel.restype = None
        L.ora_select_channels_rel.argtypes = [ctypes.c_int, _u16p, _f32p, ctypes.c_int, _u8p,
                                              _u8p]
        L.ora_query_relevance.restype = None
        L.ora_query_relevance.argtypes = [ctypes.c_int] * 4 + [_u16p, _f32p]
        L.ora_quantize_page_rel.restype = ctypes.c_int
        L.ora_quantize_page_rel.argtypes = [ctypes.c_int, ctypes.c_int, _u16p, _u16p, _f32p,
                                            _u8p, _u8p, _u8p]
        L.ora_num_threads.restype = ctypes.c_int
        L.ora_num_threads.argtypes = []
        L.ora_prefill_attention.argtypes = [ctypes.c_int] * 4 + [_u16p, _u16p, _u16p,
                                                                 ctypes.c_double, _f64p, _f64p]
        L.ora_select_tokens.argtypes = [ctypes.c_int, _f64p, ctypes.c_int, ctypes.c_int, _i32p]
        L.ora_quantize_groups.argtypes = [ctypes.c_int, _u16p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, _u16p, _u16p, _u8p]
        L.ora_prefill_rows.argtypes = [ctypes.c_int] * 4 + [_u16p, _u16p, _u16p, ctypes.c_double,
                                                            ctypes.c_int, _i32p, _f64p]
        self.L = L

    # -- stored dtypes -----------------------------------------------------
    def decode(self, dt, bits):
        bits = np.asarray(bits, dtype=np.uint16)
        f = np.vectorize(lambda h: self.L.ora_decode(dt, int(h)), otypes=[np.float64])
        return f(bits) if bits.size else bits.astype(np.float64)

    def encode(self, dt, x):
        x = np.asarray(x, dtype=np.float64)
        f = np.vectorize(lambda v: self.L.ora_encode(dt, float(v)), otypes=[np.uint16])
        return f(x) if x.size else x.astype(np.uint16)

    # -- quantizer pieces ----------------------------------------------------
    def quantize_group(self, dt, x_bits, L):
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        n = x.size
        s = np.zeros(1, np.uint16)
        z = np.zeros(1, np.uint16)
        codes = np.zeros(n, np.uint8)
        self.L.ora_quantize_group(dt, _ptr(x, _u16p), n, 1, L, _ptr(s, _u16p),
                                  _ptr(z, _u16p), _ptr(codes, _u8p), 1)
        return int(s[0]), int(z[0]), codes

    def quantize_groups(self, dt, x_bits, L):
        """n groups of glen values (x_bits [n][glen] u16), each quantized on its
        own (R2) -> (scales [n] u16, zeros [n] u16, codes [n][glen] u8)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        n, glen = x.shape
        s = np.zeros(n, np.uint16)
        z = np.zeros(n, np.uint16)
        codes = np.zeros((n, glen), np.uint8)
        self.L.ora_quantize_groups(dt, _ptr(x, _u16p), n, glen, L, _ptr(s, _u16p),
                                   _ptr(z, _u16p), _ptr(codes, _u8p))
        return s, z, codes

    def select_channels(self, K_bits, k):
        K = np.ascontiguousarray(K_bits, dtype=np.uint16)
        ntok, nch = K.shape
        boosted = np.zeros(nch, np.uint8)
        idx = np.zeros(max(k, 1), np.uint8)
        self.L.ora_select_channels(_ptr(K, _u16p), ntok, nch, k, _ptr(boosted, _u8p),
                                   _ptr(idx, _u8p))
        return boosted.astype(bool), idx[:k].copy()

    # -- pages -----------------------------------------------------------------
    def page_bytes(self, k):
        return int(self.L.ora_page_bytes(k))

    def page_layout(self, k):
        out = np.zeros(9, np.int64)
        self.L.ora_page_layout(k, _ptr(out, _i64p))
        names = ["klo", "khi", "ks", "kz", "kidx", "vc", "vs", "vz", "total"]
        return dict(zip(names, (int(v) for v in out)))

    def vcode_bit(self, t, c):
        return int(self.L.ora_vcode_bit(t, c))

    def klo_bit(self, t, c):
        return int(self.L.ora_klo_bit(t, c))

    def khi_bit(self, k, t, j):
        return int(self.L.ora_khi_bit(k, t, j))

    def select_channels_rel(self, dt, K_bits, rel, k):
        """Query-aware selection of one page: K [P][D] uint16, rel [D] float32."""
        K_bits = np.ascontiguousarray(K_bits, dtype=np.uint16)
        rel = np.ascontiguousarray(rel, dtype=np.float32)
        assert K_bits.shape == (P, D) and rel.shape == (D,)
        boosted = np.zeros(D, np.uint8)
        idx = np.zeros(D, np.uint8)
        self.L.ora_select_channels_rel(dt, _ptr(K_bits, _u16p), _ptr(rel, _f32p), k,
                                       _ptr(boosted, _u8p), _ptr(idx, _u8p))
        return boosted.astype(bool), idx[:k].copy()

    def query_relevance(self, dt, q_bits, Hkv):
        """q [B][Hq][D] uint16 -> relevance [B][Hkv][D] float32."""
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        B, Hq, _ = q_bits.shape
        rel = np.zeros((B, Hkv, D), np.float32)
        self.L.ora_query_relevance(dt, B, Hq, Hkv, _ptr(q_bits, _u16p), _ptr(rel, _f32p))
        return rel

    def quantize_page(self, dt, k, Kp, Vp, rel=None):
        """Kp, Vp: [P][D] uint16 -> (page bytes, 4-bit-or-2-bit Key codes, Value codes).
        rel ([D] float32): query-aware channel selection instead of magnitude."""
        Kp = np.ascontiguousarray(Kp, dtype=np.uint16)
        Vp = np.ascontiguousarray(Vp, dtype=np.uint16)
        assert Kp.shape == (P, D) and Vp.shape == (P, D)
        page = np.zeros(self.page_bytes(k), np.uint8)
        kc = np.zeros((P, D), np.uint8)
        vc = np.zeros((P, D), np.uint8)
        if rel is not None:
            rel = np.ascontiguousarray(rel, dtype=np.float32)
            assert rel.shape == (D,)
            rc = self.L.ora_quantize_page_rel(dt, k, _ptr(Kp, _u16p), _ptr(Vp, _u16p),
                                              _ptr(rel, _f32p), _ptr(page, _u8p),
                                              _ptr(kc, _u8p), _ptr(vc, _u8p))
        else:
            rc = self.L.ora_quantize_page(dt, k, _ptr(Kp, _u16p), _ptr(Vp, _u16p),
                                          _ptr(page, _u8p), _ptr(kc, _u8p), _ptr(vc, _u8p))
        if rc:
            raise ValueError(f"ora_quantize_page failed ({rc})")
        return page, kc, vc

    def unpack_page(self, dt, k, page):
        page = np.ascontiguousarray(page, dtype=np.uint8)
        out = dict(kcode=np.zeros((P, D), np.uint8), klo=np.zeros((P, D), np.uint8),
                   khi=np.zeros((P, max(k, 1)), np.uint8), vcode=np.zeros((P, D), np.uint8),
                   ks=np.zeros((P // GK, D), np.uint16), kz=np.zeros((P // GK, D), np.uint16),
                   vs=np.zeros((D // GV, P), np.uint16), vz=np.zeros((D // GV, P), np.uint16),
                   idx=np.zeros(max(k, 1), np.uint8))
        rc = self.L.ora_unpack_page(
            dt, k, _ptr(page, _u8p), _ptr(out["kcode"], _u8p), _ptr(out["klo"], _u8p),
            _ptr(out["khi"], _u8p), _ptr(out["vcode"], _u8p), _ptr(out["ks"], _u16p),
            _ptr(out["kz"], _u16p), _ptr(out["vs"], _u16p), _ptr(out["vz"], _u16p),
            _ptr(out["idx"], _u8p))
        if rc:
            raise ValueError(f"ora_unpack_page failed ({rc})")
        out["khi"] = out["khi"][:, :k]
        out["idx"] = out["idx"][:k]
        return out

    def dequantize_page(self, dt, k, page):
        page = np.ascontiguousarray(page, dtype=np.uint8)
        Kh = np.zeros((P, D), np.float64)
        Vh = np.zeros((P, D), np.float64)
        rc = self.L.ora_dequantize_page(dt, k, _ptr(page, _u8p), _ptr(Kh, _f64p),
                                        _ptr(Vh, _f64p))
        if rc:
            raise ValueError(f"ora_dequantize_page failed ({rc})")
        return Kh, Vh

    def attention(self, dt, k, pages, kres, vres, q, n_pages, n_res, scale,
                  units=None):
        """pages [B][Hkv][max_pages][page_bytes] u8; kres, vres [B][Hkv][R][D] u16;
        q [B][Hq][D] u16 -> out [B][Hq][D] float64 (NaN outside `units`)."""
        pages = np.ascontiguousarray(pages, dtype=np.uint8)
        kres = np.ascontiguousarray(kres, dtype=np.uint16)
        vres = np.ascontiguousarray(vres, dtype=np.uint16)
        q = np.ascontiguousarray(q, dtype=np.uint16)
        B, Hkv, max_pages, pb = pages.shape
        Hq = q.shape[1]
        assert pb == self.page_bytes(k) and kres.shape == (B, Hkv, R, D)
        assert q.shape == (B, Hq, D)
        out = np.full((B, Hq, D), np.nan, np.float64)
        u0, u1 = (0, B * Hkv) if units is None else units
        rc = self.L.ora_attention(dt, k, B, Hq, Hkv, max_pages, n_pages, n_res,
                                  _ptr(pages, _u8p), _ptr(kres, _u16p), _ptr(vres, _u16p),
                                  _ptr(q, _u16p), float(scale), _ptr(out, _f64p), u0, u1)
        if rc:
            raise ValueError(f"ora_attention failed ({rc})")
        return out

    def num_threads(self):
        return int(self.L.ora_num_threads())

    def prefill_attention(self, dt, q, k, v, scale):
        """Causal prefill attention of one sequence (R20, R21): q [Hq][T][D],
        k, v [Hkv][T][D] u16 -> (out [Hq][T][D] float64, score [Hkv][T] float64)."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        Hq, T, d = q.shape
        Hkv = k.shape[0]
        assert d == D and k.shape == (Hkv, T, D) and v.shape == k.shape
        out = np.empty((Hq, T, D), np.float64)
        score = np.empty((Hkv, T), np.float64)
        rc = self.L.ora_prefill_attention(dt, T, Hq, Hkv, _ptr(q, _u16p), _ptr(k, _u16p),
                                          _ptr(v, _u16p), float(scale), _ptr(out, _f64p),
                                          _ptr(score, _f64p))
        if rc:
            raise ValueError(f"ora_prefill_attention failed ({rc})")
        return out, score

    def prefill_rows(self, dt, q, k, v, scale, rows):
        """Causal prefill attention output of the query positions `rows` only
        (R20): q [Hq][T][D], k, v [Hkv][T][D] u16 -> out [Hq][len(rows)][D]
        float64."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        Hq, T, d = q.shape
        Hkv = k.shape[0]
        assert d == D and k.shape == (Hkv, T, D) and v.shape == k.shape
        out = np.empty((Hq, len(rows), D), np.float64)
        rc = self.L.ora_prefill_rows(dt, T, Hq, Hkv, _ptr(q, _u16p), _ptr(k, _u16p),
                                     _ptr(v, _u16p), float(scale), len(rows), _ptr(rows, _i32p),
                                     _ptr(out, _f64p))
        if rc:
            raise ValueError(f"ora_prefill_rows failed ({rc})")
        return out

    def select_tokens(self, score, heavy, recent):
        """R22: kept positions (ascending) of one KV head's scores [T]."""
        score = np.ascontiguousarray(score, dtype=np.float64)
        T = score.shape[0]
        keep = np.empty(max(T, 1), np.int32)
        n = self.L.ora_select_tokens(T, _ptr(score, _f64p), heavy, recent, _ptr(keep, _i32p))
        if n < 0:
            raise ValueError(f"ora_select_tokens failed ({n})")
        return keep[:n].copy()


_default = None


def lib():
    """The oracle proper (built on first use if no library exists)."""
    global _default
    if _default is None:
        _default = OracleLib(_build.ensure_built())
    return _default


def planted(n):
    """A copy of the oracle with mistake n planted (tests only)."""
    return OracleLib(_build.build(plant=n))


class OracleCache:
    """Host model of one quantized KV cache (flush-before-insert window).

    Readings: KIVI explainer section 3 (full-precision residual part,
    streaming append); page = 128 tokens; the window holds up to 128 exact
    tokens and a full window is quantized into a page before the next insert.
    """

    def __init__(self, dtype, B, Hq, Hkv, k, max_pages, scale=None, ora=None):
        self.ora = ora or lib()
        self.dt, self.B, self.Hq, self.Hkv, self.k = dtype, B, Hq, Hkv, k
        self.max_pages = max_pages
        self.scale = 1.0 / np.sqrt(D) if scale is None or scale <= 0 else float(scale)
        self.pb = self.ora.page_bytes(k)
        self.pages = np.zeros((B, Hkv, max_pages, self.pb), np.uint8)
        self.kres = np.zeros((B, Hkv, R, D), np.uint16)
        self.vres = np.zeros((B, Hkv, R, D), np.uint16)
        self.n_pages = 0
        self.n_res = 0
        self.rel = None  # [B][Hkv][D] float32: query-aware selection for later pages

    def _rel(self, b, h):
        return None if self.rel is None else self.rel[b, h]

    def quantize_pages(self, K, V):
        """K, V: [B][Hkv][n*P][D] uint16; appends n pages per sequence."""
        if self.n_res != 0:
            raise ValueError("bulk page quantization needs an empty residual window")
        n = K.shape[2] // P
        assert K.shape == (self.B, self.Hkv, n * P, D) and V.shape == K.shape
        if self.n_pages + n > self.max_pages:
            raise ValueError("capacity")
        for b in range(self.B):
            for h in range(self.Hkv):
                for p in range(n):
                    sl = slice(p * P, (p + 1) * P)
                    page, _, _ = self.ora.quantize_page(self.dt, self.k, K[b, h, sl], V[b, h, sl],
                                                        self._rel(b, h))
                    self.pages[b, h, self.n_pages + p] = page
        self.n_pages += n

    def append(self, k_t, v_t):
        """k_t, v_t: [B][Hkv][D] uint16.  Returns True when the window was flushed."""
        flushed = False
        if self.n_res == R:
            if self.n_pages + 1 > self.max_pages:
                raise ValueError("capacity")
            for b in range(self.B):
                for h in range(self.Hkv):
                    page, _, _ = self.ora.quantize_page(self.dt, self.k, self.kres[b, h],
                                                        self.vres[b, h], self._rel(b, h))
                    self.pages[b, h, self.n_pages] = page
            self.n_pages += 1
            self.n_res = 0
            flushed = True
        self.kres[:, :, self.n_res] = k_t
        self.vres[:, :, self.n_res] = v_t
        self.n_res += 1
        return flushed

    def attention(self, q, units=None):
        return self.ora.attention(self.dt, self.k, self.pages, self.kres, self.vres, q,
                                  self.n_pages, self.n_res, self.scale, units=units)
