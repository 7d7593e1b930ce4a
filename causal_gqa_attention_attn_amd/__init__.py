"""Python binding of libgqa (include/gqa.h): masked causal grouped-query
attention with a paged KV cache on an AMD Instinct MI355X (gfx950).

The functions carry the C names and only marshal arguments: torch tensors
become ``gqa_tensor`` descriptors (device pointer, dtype, shape, strides),
host integer arrays become contiguous numpy buffers, and the stream is torch's
current HIP stream unless one is given.  Every step of the computation runs in
the HIP kernels of the library; if ``libgqa.so`` is missing, importing this
package raises ImportError (there is no fallback).

``PagedCache`` is a convenience owner of the caller-side device buffers (pools,
block table, rotation table) allocated with torch; it reads nothing back.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgqa.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run python causal_gqa_attention_attn_amd/build.py")

_lib = ctypes.CDLL(_LIB_PATH)

F32, BF16 = 0, 1
STATUS = {0: "OK", -1: "ARG", -2: "SHAPE", -3: "DTYPE", -4: "MASK", -5: "POSITION",
          -6: "CACHE", -7: "OUT_OF_PAGES", -8: "UNSUPPORTED", -9: "HIP", -10: "DEVICE"}
EXPORTS = ["gqa_cache_buffer_sizes", "gqa_cache_create", "gqa_cache_destroy", "kv_cache_append",
           "gqa_prefill", "gqa_attention", "gqa_decode", "gqa_decode_step", "gqa_decode_step_noalloc",
           "kv_cache_truncate", "kv_cache_fork", "kv_cache_remap", "gqa_cache_length",
           "gqa_cache_page_table", "gqa_cache_free_pages", "gqa_cache_check", "gqa_workspace_size",
           "gqa_attention_workspace_size", "gqa_workspace_status", "gqa_set_merge_wait",
           "gqa_prefix_index_create", "gqa_prefix_index_destroy",
           "gqa_prefix_index_insert", "gqa_prefix_index_remove", "gqa_prefix_index_match",
           "gqa_last_error"]


class GqaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.name = STATUS.get(code, str(code))
        super().__init__(f"{where}: GQA_ERR_{self.name}: {gqa_last_error()}")


class gqa_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class gqa_cache_config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_style", ctypes.c_int32), ("max_position", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("window", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_TP = ctypes.POINTER(gqa_tensor)
_sig = {
    "gqa_cache_buffer_sizes": [ctypes.POINTER(gqa_cache_config), ctypes.POINTER(ctypes.c_size_t),
                               ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                               ctypes.POINTER(ctypes.c_size_t)],
    "gqa_cache_create": [ctypes.POINTER(gqa_cache_config), _P, _P, _P, _P, _P, ctypes.POINTER(_P)],
    "gqa_cache_destroy": [_P],
    "kv_cache_append": [_P, ctypes.c_int32, ctypes.c_int32, _P, _TP, _TP, _P, _P, _P],
    "gqa_prefill": [_P, ctypes.c_int32, ctypes.c_int32, _P, _TP, _TP, _TP, _P, _P, _TP, _P,
                    ctypes.c_size_t, _P],
    "gqa_attention": [_P, ctypes.c_int32, ctypes.c_int32, _P, _TP, _P, _P, _TP, _P, ctypes.c_size_t, _P],
    "gqa_decode": [_P, ctypes.c_int32, ctypes.c_int32, _P, _TP, _P, _TP, _P, ctypes.c_size_t, _P],
    "gqa_decode_step": [_P, ctypes.c_int32, ctypes.c_int32, _P, _TP, _TP, _TP, _TP, _P, ctypes.c_size_t, _P],
    "gqa_decode_step_noalloc": [_P, ctypes.c_int32, ctypes.c_int32, _P, _TP, _TP, _TP, _TP, _P],
    "kv_cache_truncate": [_P, ctypes.c_int32, ctypes.c_int32],
    "kv_cache_fork": [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32],
    "gqa_prefix_index_create": [_P],
    "gqa_prefix_index_destroy": [_P],
    "gqa_prefix_index_insert": [_P, ctypes.c_int32, _P, ctypes.c_int32],
    "gqa_prefix_index_remove": [_P, ctypes.c_int32],
    "gqa_prefix_index_match": [_P, _P, ctypes.c_int32, _P, _P],
    "kv_cache_remap": [_P, ctypes.c_int32, _P, _P, _P],
    "gqa_cache_length": [_P, ctypes.c_int32, ctypes.c_int32, _I32P],
    "gqa_cache_page_table": [_P, ctypes.c_int32, _P, ctypes.c_int32, _I32P],
    "gqa_cache_free_pages": [_P, _I32P],
    "gqa_cache_check": [_P],
    "gqa_workspace_size": [_P, ctypes.c_int32, ctypes.c_int32],
    "gqa_attention_workspace_size": [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32],
    "gqa_workspace_status": [_P, _P, ctypes.c_size_t, ctypes.c_int32, _P],
    "gqa_set_merge_wait": [ctypes.c_int32, ctypes.c_int32],
    "gqa_last_error": [],
}
for _name, _args in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int32
_lib.gqa_workspace_size.restype = ctypes.c_size_t
_lib.gqa_attention_workspace_size.restype = ctypes.c_size_t
_lib.gqa_last_error.restype = ctypes.c_char_p


def _check(status: int, where: str):
    if status != 0:
        raise GqaError(status, where)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    return 99


def _tensor(t: torch.Tensor) -> gqa_tensor:
    if t.dim() != 4:
        raise ValueError("tensors crossing the boundary are 4-D")
    d = gqa_tensor()
    d.data = t.data_ptr()
    d.dtype = _dtype_code(t.dtype)
    for i in range(4):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _host_i32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _host_u8(x):
    if isinstance(x, torch.Tensor):
        x = x.cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.uint8))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return None


def _cfg(**kw) -> gqa_cache_config:
    c = gqa_cache_config()
    for k, v in kw.items():
        setattr(c, k, v)
    return c


# ---------------------------------------------------------------- C entry points

def gqa_cache_buffer_sizes(cfg: gqa_cache_config):
    out = [ctypes.c_size_t() for _ in range(4)]
    _check(_lib.gqa_cache_buffer_sizes(ctypes.byref(cfg), *[ctypes.byref(o) for o in out]),
           "gqa_cache_buffer_sizes")
    return tuple(o.value for o in out)


def gqa_cache_create(cfg, k_pool, v_pool, page_table, rope_table, free_list_order=None):
    handle = ctypes.c_void_p()
    order = None if free_list_order is None else _host_i32(free_list_order)
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(_lib.gqa_cache_create(ctypes.byref(cfg), ptr(k_pool), ptr(v_pool), ptr(page_table),
                                 ptr(rope_table), None if order is None else _ptr(order),
                                 ctypes.byref(handle)), "gqa_cache_create")
    return handle


def gqa_cache_destroy(handle):
    _check(_lib.gqa_cache_destroy(handle), "gqa_cache_destroy")


def kv_cache_append(handle, layer, seq_ids, K, V, valid_mask, positions, stream=None):
    ids = _host_i32(seq_ids)
    m, p = _host_u8(valid_mask), _host_i32(positions)
    tk, tv = _tensor(K), _tensor(V)
    _check(_lib.kv_cache_append(handle, layer, len(ids), _ptr(ids), ctypes.byref(tk), ctypes.byref(tv),
                                _ptr(m), _ptr(p), _stream(stream)), "kv_cache_append")


def gqa_prefill(handle, layer, seq_ids, Q, K, V, valid_mask, positions, O, workspace=None, stream=None):
    ids = _host_i32(seq_ids)
    m, p = _host_u8(valid_mask), _host_i32(positions)
    tq, tk, tv, to = _tensor(Q), _tensor(K), _tensor(V), _tensor(O)
    ws = None if workspace is None else workspace.data_ptr()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqa_prefill(handle, layer, len(ids), _ptr(ids), ctypes.byref(tq), ctypes.byref(tk),
                            ctypes.byref(tv), _ptr(m), _ptr(p), ctypes.byref(to), ws, nbytes,
                            _stream(stream)), "gqa_prefill")


def gqa_attention(handle, layer, seq_ids, Q, valid_mask, positions, O, workspace=None, stream=None):
    ids = _host_i32(seq_ids)
    m, p = _host_u8(valid_mask), _host_i32(positions)
    tq, to = _tensor(Q), _tensor(O)
    ws = None if workspace is None else workspace.data_ptr()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqa_attention(handle, layer, len(ids), _ptr(ids), ctypes.byref(tq), _ptr(m), _ptr(p),
                              ctypes.byref(to), ws, nbytes, _stream(stream)), "gqa_attention")


def gqa_decode(handle, layer, seq_ids, q, valid_lengths, o, workspace=None, stream=None):
    ids = _host_i32(seq_ids)
    lens = _host_i32(valid_lengths)
    tq, to = _tensor(q), _tensor(o)
    ws = None if workspace is None else workspace.data_ptr()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqa_decode(handle, layer, len(ids), _ptr(ids), ctypes.byref(tq), _ptr(lens),
                           ctypes.byref(to), ws, nbytes, _stream(stream)), "gqa_decode")


def gqa_decode_step(handle, layer, seq_ids, q, k_new, v_new, o, workspace=None, stream=None):
    ids = _host_i32(seq_ids)
    tq, tk, tv, to = _tensor(q), _tensor(k_new), _tensor(v_new), _tensor(o)
    ws = None if workspace is None else workspace.data_ptr()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqa_decode_step(handle, layer, len(ids), _ptr(ids), ctypes.byref(tq), ctypes.byref(tk),
                                ctypes.byref(tv), ctypes.byref(to), ws, nbytes, _stream(stream)), "gqa_decode_step")


def gqa_decode_step_noalloc(handle, layer, seq_ids, q, k_new, v_new, o, stream=None):
    ids = _host_i32(seq_ids)
    tq, tk, tv, to = _tensor(q), _tensor(k_new), _tensor(v_new), _tensor(o)
    _check(_lib.gqa_decode_step_noalloc(handle, layer, len(ids), _ptr(ids), ctypes.byref(tq), ctypes.byref(tk),
                                        ctypes.byref(tv), ctypes.byref(to), _stream(stream)),
           "gqa_decode_step_noalloc")


def kv_cache_truncate(handle, seq_id, m):
    _check(_lib.kv_cache_truncate(handle, seq_id, m), "kv_cache_truncate")


def kv_cache_fork(handle, src_seq, dst_seq, m):
    _check(_lib.kv_cache_fork(handle, src_seq, dst_seq, m), "kv_cache_fork")


class PrefixIndex:
    """Host radix tree over recorded requests' token ids (gqa_prefix_index_*)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(_lib.gqa_prefix_index_create(ctypes.byref(h)), "gqa_prefix_index_create")
        self.handle = h

    def insert(self, seq, tokens):
        t = _host_i32(tokens)
        _check(_lib.gqa_prefix_index_insert(self.handle, seq, _ptr(t), t.size), "gqa_prefix_index_insert")

    def remove(self, seq):
        _check(_lib.gqa_prefix_index_remove(self.handle, seq), "gqa_prefix_index_remove")

    def match(self, tokens):
        t = _host_i32(tokens)
        s, m = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.gqa_prefix_index_match(self.handle, _ptr(t), t.size, ctypes.byref(s), ctypes.byref(m)),
               "gqa_prefix_index_match")
        return s.value, m.value

    def close(self):
        if self.handle:
            _lib.gqa_prefix_index_destroy(self.handle)
            self.handle = None


def kv_cache_remap(handle, src_pages, dst_pages, stream=None):
    s, d = _host_i32(src_pages), _host_i32(dst_pages)
    if s.size != d.size:
        raise ValueError("src and dst differ in length")
    _check(_lib.kv_cache_remap(handle, s.size, _ptr(s), _ptr(d), _stream(stream)), "kv_cache_remap")


def gqa_cache_length(handle, seq_id, layer) -> int:
    out = ctypes.c_int32()
    _check(_lib.gqa_cache_length(handle, seq_id, layer, ctypes.byref(out)), "gqa_cache_length")
    return out.value


def gqa_cache_page_table(handle, seq_id) -> list:
    n = ctypes.c_int32()
    _lib.gqa_cache_page_table(handle, seq_id, None, 0, ctypes.byref(n))
    buf = np.zeros(max(1, n.value), dtype=np.int32)
    _check(_lib.gqa_cache_page_table(handle, seq_id, _ptr(buf), buf.size, ctypes.byref(n)),
           "gqa_cache_page_table")
    return [int(x) for x in buf[:n.value]]


def gqa_cache_free_pages(handle) -> int:
    out = ctypes.c_int32()
    _check(_lib.gqa_cache_free_pages(handle, ctypes.byref(out)), "gqa_cache_free_pages")
    return out.value


def gqa_cache_check(handle):
    _check(_lib.gqa_cache_check(handle), "gqa_cache_check")


def gqa_workspace_size(handle, B, Hq) -> int:
    return int(_lib.gqa_workspace_size(handle, B, Hq))


def gqa_attention_workspace_size(handle, B, Hq, n) -> int:
    return int(_lib.gqa_attention_workspace_size(handle, B, Hq, n))


def gqa_workspace_status(handle, workspace, clear=False, stream=None):
    """Raises GqaError (GQA_ERR_DEVICE) if a split combine using this workspace
    gave up since the status was last cleared; clear=True resets it after the
    read.  workspace None: the static scratch of gqa_decode_step_noalloc."""
    ptr = None if workspace is None else workspace.data_ptr()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqa_workspace_status(handle, ptr, nbytes, 1 if clear else 0, _stream(stream)),
           "gqa_workspace_status")


def gqa_set_merge_wait(polls, unreachable=False):
    _check(_lib.gqa_set_merge_wait(polls, 1 if unreachable else 0), "gqa_set_merge_wait")


def gqa_last_error() -> str:
    return _lib.gqa_last_error().decode()


# ---------------------------------------------------------------- buffer owner

class PagedCache:
    """Owns the caller-side device buffers of one cache and its handle."""

    def __init__(self, num_layers, num_kv_heads, head_dim, num_pages, max_seqs, max_pages_per_seq,
                 dtype=torch.bfloat16, rope_theta=0.0, max_position=None, free_list_order=None,
                 device="cuda", page_size=16, window=0):
        self.dtype = dtype
        self.cfg = _cfg(num_layers=num_layers, num_kv_heads=num_kv_heads, head_dim=head_dim,
                        page_size=page_size, num_pages=num_pages, max_seqs=max_seqs,
                        max_pages_per_seq=max_pages_per_seq, dtype=_dtype_code(dtype),
                        rope_style=1 if rope_theta else 0,
                        max_position=max_position if max_position else max_pages_per_seq * page_size,
                        rope_theta=float(rope_theta), window=int(window))
        kb, vb, tb, rb = gqa_cache_buffer_sizes(self.cfg)
        elt = 2 if dtype == torch.bfloat16 else 4
        self.k_pool = torch.empty(kb // elt, dtype=dtype, device=device)
        self.v_pool = torch.empty(vb // elt, dtype=dtype, device=device)
        self.page_table = torch.zeros(tb // 4, dtype=torch.int32, device=device)
        self.rope_table = torch.empty(max(1, rb // 4), dtype=torch.float32, device=device) if rb else None
        self.handle = gqa_cache_create(self.cfg, self.k_pool, self.v_pool, self.page_table,
                                       self.rope_table, free_list_order)
        self.L, self.Hkv, self.d, self.P = num_layers, num_kv_heads, head_dim, page_size
        self.num_pages, self.max_pages_per_seq = num_pages, max_pages_per_seq
        self.window = int(window)

    def close(self):
        if self.handle is not None:
            gqa_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
