"""ctypes binding of libkvq.so (include/kvq.h), same entry-point names.

Argument marshalling only: tensors become device pointers, the torch stream
becomes a hipStream_t, negative return codes become `KvqError`.  Every step of
the path runs in the library's HIP kernels.  Importing this module raises if
the library has not been built.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
_L = ctypes.CDLL(LIB_PATH)

KVQ_F16, KVQ_BF16 = 0, 1
KVQ_DEVICE_STATE_WORDS = 8
ERRORS = {-1: "KVQ_EINVAL", -2: "KVQ_ECAPACITY", -3: "KVQ_ESTATE", -4: "KVQ_EEMPTY",
          -5: "KVQ_EWORKSPACE", -6: "KVQ_EALIGN", -7: "KVQ_EHIP"}
EXPORTS = ["kvq_cache_bytes", "kvq_page_bytes", "kvq_cache_create", "kvq_cache_destroy",
           "kvq_quantize_page", "kvq_append_token", "kvq_decode_workspace_bytes",
           "kvq_decode_attention", "kvq_append_decode", "kvq_set_decode_splits",
           "kvq_get_decode_splits",
           "kvq_get_state", "kvq_set_state", "kvq_page_offset", "kvq_residual_offset",
           "kvq_quantize_groups", "kvq_set_kernel_events", "kvq_strerror",
           "kvq_pool_bytes", "kvq_pool_create", "kvq_pool_destroy", "kvq_pool_prefill",
           "kvq_pool_append", "kvq_pool_decode_workspace_bytes", "kvq_pool_decode_attention",
           "kvq_pool_append_decode", "kvq_pool_release", "kvq_pool_get_seq",
           "kvq_pool_block_of", "kvq_pool_free_blocks", "kvq_pool_page_offset",
           "kvq_pool_window_offset", "kvq_pool_table_offset", "kvq_pool_set_kernel_events",
           "kvq_set_channel_relevance", "kvq_query_relevance", "kvq_pool_set_channel_relevance",
           "kvq_device_state_init", "kvq_append_decode_device",
           "kvq_prefill_workspace_bytes", "kvq_prefill_select", "kvq_prefill_set_kernel_events",
           "kvq_prefill_set_max_key_splits", "kvq_check_decode_plan",
           "kvq_pool_check_decode_plan", "kvq_decode_attention_noalloc", "kvq_probe_bandwidth"]


class KvqError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        self.name = ERRORS.get(code, str(code))
        msg = _L.kvq_strerror(code).decode()
        super().__init__(f"{where}: {self.name} ({msg})")


class KvqConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32), ("key_group_tokens", ctypes.c_int32),
                ("value_group_channels", ctypes.c_int32), ("residual_tokens", ctypes.c_int32),
                ("boost_channels", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


def config(batch, num_q_heads, num_kv_heads, boost_channels, max_pages, dtype,
           softmax_scale=0.0, head_dim=128, page_tokens=128, key_group_tokens=32,
           value_group_channels=32, residual_tokens=128):
    return KvqConfig(batch, num_q_heads, num_kv_heads, head_dim, page_tokens,
                     key_group_tokens, value_group_channels, residual_tokens,
                     boost_channels, max_pages, dtype, softmax_scale)


_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i32 = ctypes.c_int32
_cfgp = ctypes.POINTER(KvqConfig)
_SIG = {
    "kvq_cache_bytes": [_cfgp, ctypes.POINTER(_sz)],
    "kvq_page_bytes": [_cfgp, ctypes.POINTER(_sz)],
    "kvq_cache_create": [_cfgp, _vp, _sz, ctypes.POINTER(_vp)],
    "kvq_cache_destroy": [_vp],
    "kvq_quantize_page": [_vp, _vp, _vp, _i32, _vp],
    "kvq_append_token": [_vp, _vp, _vp, _vp, ctypes.POINTER(_i32)],
    "kvq_decode_workspace_bytes": [_vp, ctypes.POINTER(_sz)],
    "kvq_decode_attention": [_vp, _vp, _vp, _vp, _sz, _vp],
    "kvq_append_decode": [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, ctypes.POINTER(_i32)],
    "kvq_set_decode_splits": [_vp, _i32],
    "kvq_get_decode_splits": [_vp, ctypes.POINTER(_i32)],
    "kvq_get_state": [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32)],
    "kvq_set_state": [_vp, _i32, _i32],
    "kvq_page_offset": [_vp, _i32, _i32, _i32, ctypes.POINTER(_sz)],
    "kvq_residual_offset": [_vp, _i32, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
    "kvq_quantize_groups": [_i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp],
    "kvq_set_kernel_events": [_vp, _vp, _vp],
    "kvq_pool_bytes": [_cfgp, _i32, ctypes.POINTER(_sz)],
    "kvq_pool_create": [_cfgp, _i32, _vp, _sz, ctypes.POINTER(_vp)],
    "kvq_pool_destroy": [_vp],
    "kvq_pool_prefill": [_vp, _i32, _vp, _vp, _i32, _vp],
    "kvq_pool_append": [_vp, _vp, _vp, _vp, ctypes.POINTER(_i32)],
    "kvq_pool_decode_workspace_bytes": [_vp, ctypes.POINTER(_sz)],
    "kvq_pool_decode_attention": [_vp, _vp, _vp, _vp, _sz, _vp],
    "kvq_pool_append_decode": [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, ctypes.POINTER(_i32)],
    "kvq_pool_release": [_vp, _i32],
    "kvq_pool_get_seq": [_vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                         ctypes.POINTER(_i32)],
    "kvq_pool_block_of": [_vp, _i32, _i32, ctypes.POINTER(_i32)],
    "kvq_pool_free_blocks": [_vp, ctypes.POINTER(_i32)],
    "kvq_pool_page_offset": [_vp, _i32, _i32, ctypes.POINTER(_sz)],
    "kvq_pool_window_offset": [_vp, _i32, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
    "kvq_pool_table_offset": [_vp, ctypes.POINTER(_sz)],
    "kvq_pool_set_kernel_events": [_vp, _vp, _vp],
    "kvq_prefill_set_kernel_events": [_vp, _vp],
    "kvq_prefill_set_max_key_splits": [_i32],
    "kvq_decode_attention_noalloc": [_vp, _vp, _vp, _vp],
    "kvq_probe_bandwidth": [_i32, _vp, _vp, _sz, _vp],
    "kvq_check_decode_plan": [_vp, _i32, _i32, _sz, ctypes.c_char_p, _sz],
    "kvq_pool_check_decode_plan": [_vp, _i32, _i32, _sz, ctypes.c_char_p, _sz],
    "kvq_set_channel_relevance": [_vp, _vp],
    "kvq_query_relevance": [_i32, _i32, _i32, _i32, _vp, _vp, _vp],
    "kvq_pool_set_channel_relevance": [_vp, _vp],
    "kvq_device_state_init": [_vp, _vp, _vp],
    "kvq_append_decode_device": [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp],
    "kvq_prefill_workspace_bytes": [_i32, _i32, _i32, ctypes.POINTER(_sz)],
    "kvq_prefill_select": [_i32, _i32, _i32, _i32, ctypes.c_float, _vp, _vp, _vp, _i32, _i32,
                           _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, ctypes.POINTER(_i32)],
}
for _name, _args in _SIG.items():
    _f = getattr(_L, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_L.kvq_strerror.argtypes = [ctypes.c_int]
_L.kvq_strerror.restype = ctypes.c_char_p


def _check(rc, where):
    if rc != 0:
        raise KvqError(rc, where)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# -- entry points (same names as the C ABI) ----------------------------------
def kvq_cache_bytes(cfg):
    n = _sz()
    _check(_L.kvq_cache_bytes(ctypes.byref(cfg), ctypes.byref(n)), "kvq_cache_bytes")
    return n.value


def kvq_page_bytes(cfg):
    n = _sz()
    _check(_L.kvq_page_bytes(ctypes.byref(cfg), ctypes.byref(n)), "kvq_page_bytes")
    return n.value


def kvq_cache_create(cfg, dev_mem, nbytes):
    h = _vp()
    _check(_L.kvq_cache_create(ctypes.byref(cfg), _ptr(dev_mem), nbytes, ctypes.byref(h)),
           "kvq_cache_create")
    return h.value


def kvq_cache_destroy(handle):
    _check(_L.kvq_cache_destroy(handle), "kvq_cache_destroy")


def kvq_quantize_page(handle, k, v, n_pages, stream=None):
    _check(_L.kvq_quantize_page(handle, _ptr(k), _ptr(v), n_pages, _stream(stream)),
           "kvq_quantize_page")


def kvq_append_token(handle, k, v, stream=None):
    f = _i32()
    _check(_L.kvq_append_token(handle, _ptr(k), _ptr(v), _stream(stream), ctypes.byref(f)),
           "kvq_append_token")
    return bool(f.value)


def kvq_decode_workspace_bytes(handle):
    n = _sz()
    _check(_L.kvq_decode_workspace_bytes(handle, ctypes.byref(n)), "kvq_decode_workspace_bytes")
    return n.value


def kvq_decode_attention(handle, q, out, workspace, ws_bytes, stream=None):
    _check(_L.kvq_decode_attention(handle, _ptr(q), _ptr(out), _ptr(workspace), ws_bytes,
                                   _stream(stream)), "kvq_decode_attention")


def kvq_append_decode(handle, k, v, q, out, workspace, ws_bytes, stream=None):
    f = _i32()
    _check(_L.kvq_append_decode(handle, _ptr(k), _ptr(v), _ptr(q), _ptr(out), _ptr(workspace),
                                ws_bytes, _stream(stream), ctypes.byref(f)), "kvq_append_decode")
    return bool(f.value)


def kvq_device_state_init(handle, dev_state, stream=None):
    _check(_L.kvq_device_state_init(handle, _ptr(dev_state), _stream(stream)),
           "kvq_device_state_init")


def kvq_append_decode_device(handle, k, v, q, out, workspace, ws_bytes, dev_state, stream=None):
    _check(_L.kvq_append_decode_device(handle, _ptr(k), _ptr(v), _ptr(q), _ptr(out),
                                       _ptr(workspace), ws_bytes, _ptr(dev_state),
                                       _stream(stream)), "kvq_append_decode_device")


def kvq_set_decode_splits(handle, splits):
    _check(_L.kvq_set_decode_splits(handle, splits), "kvq_set_decode_splits")


def kvq_get_decode_splits(handle):
    s = _i32()
    _check(_L.kvq_get_decode_splits(handle, ctypes.byref(s)), "kvq_get_decode_splits")
    return s.value


def kvq_get_state(handle):
    a, b = _i32(), _i32()
    _check(_L.kvq_get_state(handle, ctypes.byref(a), ctypes.byref(b)), "kvq_get_state")
    return a.value, b.value


def kvq_set_state(handle, n_pages, n_res):
    _check(_L.kvq_set_state(handle, n_pages, n_res), "kvq_set_state")


def kvq_page_offset(handle, b, h, page):
    o = _sz()
    _check(_L.kvq_page_offset(handle, b, h, page, ctypes.byref(o)), "kvq_page_offset")
    return o.value


def kvq_residual_offset(handle, b, h):
    ko, vo = _sz(), _sz()
    _check(_L.kvq_residual_offset(handle, b, h, ctypes.byref(ko), ctypes.byref(vo)),
           "kvq_residual_offset")
    return ko.value, vo.value


def kvq_quantize_groups(dtype, L, x, n_groups, group_len, s, z, codes, stream=None):
    _check(_L.kvq_quantize_groups(dtype, L, _ptr(x), n_groups, group_len, _ptr(s), _ptr(z),
                                  _ptr(codes), _stream(stream)), "kvq_quantize_groups")


def kvq_set_kernel_events(handle, before, after):
    _check(_L.kvq_set_kernel_events(handle, _ptr(before), _ptr(after)), "kvq_set_kernel_events")


def kvq_strerror(code):
    return _L.kvq_strerror(code).decode()


def kvq_set_channel_relevance(handle, rel):
    _check(_L.kvq_set_channel_relevance(handle, _ptr(rel)), "kvq_set_channel_relevance")


def kvq_query_relevance(dtype, batch, num_q_heads, num_kv_heads, q, rel, stream=None):
    _check(_L.kvq_query_relevance(dtype, batch, num_q_heads, num_kv_heads, _ptr(q), _ptr(rel),
                                  _stream(stream)), "kvq_query_relevance")


def kvq_prefill_workspace_bytes(T, num_q_heads, num_kv_heads):
    n = _sz()
    _check(_L.kvq_prefill_workspace_bytes(T, num_q_heads, num_kv_heads, ctypes.byref(n)),
           "kvq_prefill_workspace_bytes")
    return n.value


def kvq_prefill_select(dtype, T, num_q_heads, num_kv_heads, softmax_scale, q, k, v, heavy, recent,
                       out, score, keep, k_sel, v_sel, workspace, ws_bytes, stream=None):
    n = _i32()
    _check(_L.kvq_prefill_select(dtype, T, num_q_heads, num_kv_heads, softmax_scale, _ptr(q),
                                 _ptr(k), _ptr(v), heavy, recent, _ptr(out), _ptr(score),
                                 _ptr(keep), _ptr(k_sel), _ptr(v_sel), _ptr(workspace), ws_bytes,
                                 _stream(stream), ctypes.byref(n)), "kvq_prefill_select")
    return n.value


def prefill_select(dtype, q, k, v, heavy, recent, softmax_scale=0.0, gather=True, stream=None):
    """Allocate the outputs (torch device tensors) and run kvq_prefill_select.
    q: [Hq][T][128], k, v: [Hkv][T][128] int16 bit patterns.  Returns (out,
    score, keep, k_sel, v_sel); k_sel and v_sel are None without gather."""
    Hq, T, _ = q.shape
    Hkv = k.shape[0]
    dev = q.device
    rec = min(recent, T)
    nk = min(heavy, T - rec) + rec
    out = torch.empty(Hq, T, 128, dtype=torch.float32, device=dev)
    score = torch.empty(Hkv, T, dtype=torch.float32, device=dev)
    keep = torch.empty(Hkv, max(nk, 1), dtype=torch.int32, device=dev)
    k_sel = torch.empty(Hkv, max(nk, 1), 128, dtype=torch.int16, device=dev) if gather else None
    v_sel = torch.empty_like(k_sel) if gather else None
    wsb = kvq_prefill_workspace_bytes(T, Hq, Hkv)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    n = kvq_prefill_select(dtype, T, Hq, Hkv, softmax_scale, q, k, v, heavy, recent, out, score,
                           keep, k_sel, v_sel, ws, wsb, stream)
    assert n == nk
    return out, score, keep[:, :nk], (k_sel[:, :nk] if gather else None), \
        (v_sel[:, :nk] if gather else None)


def kvq_pool_set_channel_relevance(handle, rel):
    _check(_L.kvq_pool_set_channel_relevance(handle, _ptr(rel)),
           "kvq_pool_set_channel_relevance")


# -- block pool (variable-length batches) ---------------------------------------
def kvq_pool_bytes(cfg, n_blocks):
    n = _sz()
    _check(_L.kvq_pool_bytes(ctypes.byref(cfg), n_blocks, ctypes.byref(n)), "kvq_pool_bytes")
    return n.value


def kvq_pool_create(cfg, n_blocks, dev_mem, nbytes):
    h = _vp()
    _check(_L.kvq_pool_create(ctypes.byref(cfg), n_blocks, _ptr(dev_mem), nbytes,
                              ctypes.byref(h)), "kvq_pool_create")
    return h.value


def kvq_pool_destroy(handle):
    _check(_L.kvq_pool_destroy(handle), "kvq_pool_destroy")


def kvq_pool_prefill(handle, seq, k, v, n_tokens, stream=None):
    _check(_L.kvq_pool_prefill(handle, seq, _ptr(k), _ptr(v), n_tokens, _stream(stream)),
           "kvq_pool_prefill")


def kvq_pool_append(handle, k, v, stream=None):
    f = _i32()
    _check(_L.kvq_pool_append(handle, _ptr(k), _ptr(v), _stream(stream), ctypes.byref(f)),
           "kvq_pool_append")
    return f.value


def kvq_pool_decode_workspace_bytes(handle):
    n = _sz()
    _check(_L.kvq_pool_decode_workspace_bytes(handle, ctypes.byref(n)),
           "kvq_pool_decode_workspace_bytes")
    return n.value


def kvq_pool_decode_attention(handle, q, out, workspace, ws_bytes, stream=None):
    _check(_L.kvq_pool_decode_attention(handle, _ptr(q), _ptr(out), _ptr(workspace), ws_bytes,
                                        _stream(stream)), "kvq_pool_decode_attention")


def kvq_pool_append_decode(handle, k, v, q, out, workspace, ws_bytes, stream=None):
    f = _i32()
    _check(_L.kvq_pool_append_decode(handle, _ptr(k), _ptr(v), _ptr(q), _ptr(out),
                                     _ptr(workspace), ws_bytes, _stream(stream),
                                     ctypes.byref(f)), "kvq_pool_append_decode")
    return f.value


def kvq_pool_release(handle, seq):
    _check(_L.kvq_pool_release(handle, seq), "kvq_pool_release")


def kvq_pool_get_seq(handle, seq):
    a, b, c = _i32(), _i32(), _i32()
    _check(_L.kvq_pool_get_seq(handle, seq, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "kvq_pool_get_seq")
    return bool(a.value), b.value, c.value


def kvq_pool_block_of(handle, seq, page):
    b = _i32()
    _check(_L.kvq_pool_block_of(handle, seq, page, ctypes.byref(b)), "kvq_pool_block_of")
    return b.value


def kvq_pool_free_blocks(handle):
    n = _i32()
    _check(_L.kvq_pool_free_blocks(handle, ctypes.byref(n)), "kvq_pool_free_blocks")
    return n.value


def kvq_pool_page_offset(handle, block, h):
    o = _sz()
    _check(_L.kvq_pool_page_offset(handle, block, h, ctypes.byref(o)), "kvq_pool_page_offset")
    return o.value


def kvq_pool_window_offset(handle, seq, h):
    ko, vo = _sz(), _sz()
    _check(_L.kvq_pool_window_offset(handle, seq, h, ctypes.byref(ko), ctypes.byref(vo)),
           "kvq_pool_window_offset")
    return ko.value, vo.value


def kvq_pool_table_offset(handle):
    o = _sz()
    _check(_L.kvq_pool_table_offset(handle, ctypes.byref(o)), "kvq_pool_table_offset")
    return o.value


def kvq_pool_set_kernel_events(handle, before, after):
    _check(_L.kvq_pool_set_kernel_events(handle, _ptr(before), _ptr(after)),
           "kvq_pool_set_kernel_events")


def kvq_prefill_set_kernel_events(before, after):
    """Timing hooks around the prefill attention kernel (hipEvent_t values or None)."""
    _check(_L.kvq_prefill_set_kernel_events(_ptr(before), _ptr(after)),
           "kvq_prefill_set_kernel_events")


def kvq_decode_attention_noalloc(handle, q, out, stream=None):
    _check(_L.kvq_decode_attention_noalloc(handle, _ptr(q), _ptr(out), _stream(stream)),
           "kvq_decode_attention_noalloc")


def kvq_probe_bandwidth(mode, src, dst, nbytes, stream=None):
    """Bandwidth probe: mode 0 reads src, mode 1 copies src to dst."""
    _check(_L.kvq_probe_bandwidth(mode, _ptr(src), _ptr(dst), nbytes, _stream(stream)),
           "kvq_probe_bandwidth")


def kvq_check_decode_plan(handle, mode, slots, ws_bytes):
    """Host-side extent check of a decode launch: (code, message)."""
    buf = ctypes.create_string_buffer(256)
    rc = _L.kvq_check_decode_plan(handle, mode, slots, ws_bytes, buf, len(buf))
    return rc, buf.value.decode()


def kvq_pool_check_decode_plan(handle, mode, slots, ws_bytes):
    """Host-side extent check of a pool decode launch: (code, message)."""
    buf = ctypes.create_string_buffer(256)
    rc = _L.kvq_pool_check_decode_plan(handle, mode, slots, ws_bytes, buf, len(buf))
    return rc, buf.value.decode()


def kvq_prefill_set_max_key_splits(n):
    """Cap on the prefill's key chunks (1..4), 0 = automatic."""
    _check(_L.kvq_prefill_set_max_key_splits(n), "kvq_prefill_set_max_key_splits")


# -- convenience owner of the device buffers -----------------------------------
def _torch_alloc(nbytes, device):
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


class Cache:
    """Owns a cache's device memory and workspace (torch tensors) and its handle."""

    def __init__(self, cfg, device="cuda", alloc=None):
        """alloc(nbytes, device) -> uint8 device tensor for the cache memory
        and the workspace (default: torch.empty)."""
        alloc = alloc or _torch_alloc
        self.cfg = cfg
        self.nbytes = kvq_cache_bytes(cfg)
        self.mem = alloc(self.nbytes, device)
        self.handle = kvq_cache_create(cfg, self.mem, self.nbytes)
        self.ws_bytes = kvq_decode_workspace_bytes(self.handle)
        self.ws = alloc(max(self.ws_bytes, 16), device)
        self.page_bytes = kvq_page_bytes(cfg)

    def check_plan(self, mode=0, slots=0):
        """Host-side extent check of the next decode launch (kvq_check_decode_plan)."""
        return kvq_check_decode_plan(self.handle, mode, slots, self.ws_bytes)

    def quantize_page(self, k, v, n_pages, stream=None):
        kvq_quantize_page(self.handle, k, v, n_pages, stream)

    def append_token(self, k, v, stream=None):
        return kvq_append_token(self.handle, k, v, stream)

    def decode_attention(self, q, out, stream=None):
        kvq_decode_attention(self.handle, q, out, self.ws, self.ws_bytes, stream)

    def append_decode(self, k, v, q, out, stream=None):
        return kvq_append_decode(self.handle, k, v, q, out, self.ws, self.ws_bytes, stream)

    def set_relevance(self, rel):
        """rel: [B][Hkv][128] float32 device tensor (kept alive by the caller), or None."""
        self._rel = rel
        kvq_set_channel_relevance(self.handle, rel)

    def device_state(self, stream=None):
        """A new int32[KVQ_DEVICE_STATE_WORDS] device state holding the current
        counters (a full window with a free page is flushed first)."""
        st = torch.zeros(KVQ_DEVICE_STATE_WORDS, dtype=torch.int32, device=self.mem.device)
        kvq_device_state_init(self.handle, st, stream)
        return st

    def append_decode_device(self, k, v, q, out, dev_state, stream=None):
        kvq_append_decode_device(self.handle, k, v, q, out, self.ws, self.ws_bytes, dev_state,
                                 stream)

    @property
    def state(self):
        return kvq_get_state(self.handle)

    def pages_view(self):
        """[B][Hkv][max_pages][page_bytes] uint8 view of the page region."""
        c = self.cfg
        n = c.batch * c.num_kv_heads * c.max_pages * self.page_bytes
        return self.mem[:n].view(c.batch, c.num_kv_heads, c.max_pages, self.page_bytes)

    def window_view(self):
        """K and V windows, each [B][Hkv][128][128] as int16 bit patterns."""
        c = self.cfg
        base = c.batch * c.num_kv_heads * c.max_pages * self.page_bytes
        w = self.mem[base:].view(torch.int16).view(c.batch, c.num_kv_heads, 2, 128, 128)
        return w[:, :, 0], w[:, :, 1]

    def close(self):
        if self.handle:
            kvq_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Pool:
    """Owns a block pool's device memory and workspace (torch tensors) and its handle."""

    def __init__(self, cfg, n_blocks, device="cuda", alloc=None):
        alloc = alloc or _torch_alloc
        self.cfg = cfg
        self.n_blocks = n_blocks
        self.nbytes = kvq_pool_bytes(cfg, n_blocks)
        self.mem = alloc(self.nbytes, device)
        self.handle = kvq_pool_create(cfg, n_blocks, self.mem, self.nbytes)
        self.ws_bytes = kvq_pool_decode_workspace_bytes(self.handle)
        self.ws = alloc(max(self.ws_bytes, 16), device)
        self.page_bytes = kvq_page_bytes(cfg)

    def check_plan(self, mode=0, slots=0):
        """Host-side extent check of the next decode launch (kvq_pool_check_decode_plan)."""
        return kvq_pool_check_decode_plan(self.handle, mode, slots, self.ws_bytes)

    def prefill(self, seq, k, v, stream=None):
        """k, v: [Hkv][n_tokens][128] device tensors of one sequence."""
        kvq_pool_prefill(self.handle, seq, k, v, int(k.shape[1]), stream)

    def append(self, k, v, stream=None):
        return kvq_pool_append(self.handle, k, v, stream)

    def decode_attention(self, q, out, stream=None):
        kvq_pool_decode_attention(self.handle, q, out, self.ws, self.ws_bytes, stream)

    def append_decode(self, k, v, q, out, stream=None):
        return kvq_pool_append_decode(self.handle, k, v, q, out, self.ws, self.ws_bytes, stream)

    def release(self, seq):
        kvq_pool_release(self.handle, seq)

    def set_relevance(self, rel):
        """rel: [batch][Hkv][128] float32 device tensor (kept alive by the caller), or None."""
        self._rel = rel
        kvq_pool_set_channel_relevance(self.handle, rel)

    def seq(self, seq):
        """(live, n_pages, n_res) of one slot."""
        return kvq_pool_get_seq(self.handle, seq)

    def block_of(self, seq, page):
        return kvq_pool_block_of(self.handle, seq, page)

    @property
    def free_blocks(self):
        return kvq_pool_free_blocks(self.handle)

    def page_view(self, block, h):
        o = kvq_pool_page_offset(self.handle, block, h)
        return self.mem[o:o + self.page_bytes]

    def window_view(self, seq, h):
        """K and V window of (seq, h), each [128][128] as int16 bit patterns."""
        ko, vo = kvq_pool_window_offset(self.handle, seq, h)
        n = 128 * 128 * 2
        return (self.mem[ko:ko + n].view(torch.int16).view(128, 128),
                self.mem[vo:vo + n].view(torch.int16).view(128, 128))

    def table_view(self):
        c = self.cfg
        o = kvq_pool_table_offset(self.handle)
        return self.mem[o:o + 4 * c.batch * c.max_pages].view(torch.int32).view(c.batch,
                                                                                 c.max_pages)

    def close(self):
        if self.handle:
            kvq_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
