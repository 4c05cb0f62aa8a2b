"""ctypes binding of libbitkv.so (include/bitkv.h), same names as the C ABI.

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind these calls.  torch is used for device memory and streams.
Importing this module without the built library raises immediately: there is
no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# BKV_SANITIZE=1: the sanitizer build of the same sources (host-side checks
# on the CPU; built by `python bit_kv_attention_amd/build.py --sanitize`)
LIB_PATH = os.path.join(_HERE, "libbitkv_san.so" if os.environ.get("BKV_SANITIZE") == "1" else "libbitkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python bit_kv_attention_amd/build.py`; there is no non-HIP fallback.")

# torch ships its own HIP runtime (same soname as ROCm's).  Loading torch first
# makes libbitkv.so bind to that runtime, which owns the tensors' memory and
# streams; loading the library first would put a second runtime in the process.
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)

STATUS = {0: "BKV_OK", 1: "BKV_E_NULL", 2: "BKV_E_SHAPE", 3: "BKV_E_UNSUPPORTED",
          4: "BKV_E_CAPACITY", 5: "BKV_E_WORKSPACE", 6: "BKV_E_HIP", 7: "BKV_E_ARG"}


class BitKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.bkv_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class Layout(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("batch", "n_q_heads", "n_kv_heads", "head_dim", "k_bits",
                                         "v_bits", "group", "capacity", "query_bits",
                                         "key_format")]


class CacheView(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow")]


class HybridSlot(C.Structure):
    _fields_ = [("sigma", C.c_void_p), ("idx", C.c_void_p), ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
                ("state_dev", C.c_void_p), ("idx_host", C.c_void_p), ("q_host", C.c_void_p),
                ("state_host", C.c_void_p)]


_P = C.c_void_p
_LP = C.POINTER(Layout)
_CP = C.POINTER(CacheView)
_SZ = C.POINTER(C.c_size_t)
_lib.bkv_status_string.argtypes = [C.c_int]
_lib.bkv_status_string.restype = C.c_char_p
_lib.bkv_cache_bytes.argtypes = [_LP, _SZ, _SZ, _SZ, _SZ]
_lib.bkv_workspace_bytes.argtypes = [_LP, C.c_int32, C.c_int32, _SZ]
_lib.bkv_k_meta_bytes.argtypes = [_LP, _SZ]
_lib.kv_pack_append.argtypes = [_LP, _CP, _P, _P, C.c_int32, _P, _P]
_lib.qattn_decode_approx.argtypes = [_LP, _CP, _P, _P, _P, _P, C.c_size_t, _P]
_lib.topk_select.argtypes = [_LP, _P, _P, C.c_int32, _P, _P, C.c_size_t, _P]
_lib.qattn_decode_select.argtypes = [_LP, _CP, _P, _P, C.c_int32, _P, _P, _P, C.c_size_t, C.c_int32, _P]
_lib.qattn_decode_step.argtypes = [_LP, _CP, _P, _P, _P, _P, C.c_int32, _P, _P, _P, C.c_size_t, C.c_int32, _P]
_lib.bkv_select_in_scan.argtypes = [_LP, C.c_int32, C.c_int32, C.c_int32, _P]
_lib.topk_select_window.argtypes = [_LP, _P, _P, C.c_int32, C.c_int32, _P, _P, C.c_size_t, _P]
_lib.topk_select_blocks.argtypes = [_LP, _P, _P, C.c_int32, C.c_int32, _P, _P, C.c_size_t, _P]
_lib.qattn_correct.argtypes = [_LP, _CP, _P, _P, _P, C.c_int32, _P, C.c_size_t, _P, _P]
_lib.qattn_correct_blocks.argtypes = [_LP, _CP, _P, _P, _P, C.c_int32, C.c_int32, _P, C.c_size_t, _P, _P]
_lib.qattn_hybrid_layers.argtypes = [_LP, C.c_int32, _P, _P, _P, _P, _P, C.c_int32, C.c_int32, _P, _P, C.c_int32,
                                     _P]
_lib.qattn_score_select.argtypes = [_LP, _CP, _P, _P, C.c_int32, _P, _P, _P, C.c_size_t, C.c_int32, _P]
_lib.qattn_decode_unselected.argtypes = [_LP, _CP, _P, _P, _P, C.c_int32, _P, C.c_size_t, _P]
_lib.qattn_correct_unselected.argtypes = [_LP, _CP, _P, _P, _P, C.c_int32, _P, C.c_size_t, _P, _P]
_lib.qattn_correct_hybrid.argtypes = [_LP, _CP, _P, _P, _P, C.c_int32, _P, _P, C.c_size_t, _P, _P]
_lib.qattn_exact_host.argtypes = [_LP, _P, _P, _P, _P, _P, C.c_int32, _P, C.c_int32]
_lib.qattn_decode_fused.argtypes = [_LP, _CP, _P, _P, _P, _P, C.c_int32, _P, _P, _P, _P, C.c_size_t, _P]
_lib.bkv_fused_supported.argtypes = [_LP, C.c_int32, C.c_int32, _P]
_lib.qattn_decode_fused_noalloc.argtypes = [_LP, _CP, _P, _P, _P, _P, C.c_int32, _P, _P, _P, _P]
for _f in ("bkv_cache_bytes", "bkv_k_meta_bytes", "bkv_workspace_bytes", "bkv_select_in_scan", "kv_pack_append",
           "qattn_decode_approx", "qattn_decode_select", "topk_select", "topk_select_window", "topk_select_blocks", "qattn_correct"):
    getattr(_lib, _f).restype = C.c_int

EXPORTED = ("bkv_status_string", "bkv_cache_bytes", "bkv_k_meta_bytes", "bkv_workspace_bytes", "bkv_select_in_scan",
            "kv_pack_append", "qattn_decode_approx", "qattn_decode_select", "topk_select", "topk_select_window", "topk_select_blocks",
            "qattn_correct", "qattn_correct_hybrid", "qattn_exact_host", "qattn_decode_unselected",
            "qattn_correct_unselected", "qattn_score_select", "qattn_decode_step", "qattn_decode_fused",
            "bkv_fused_supported", "qattn_decode_fused_noalloc", "qattn_correct_blocks", "qattn_hybrid_layers")


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise BitKVError(fn, st)


def _ptr(t) -> int | None:
    """Device/host address of a torch tensor (or None / an int address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_layout(batch, n_q_heads, n_kv_heads, capacity, k_bits, v_bits, head_dim=128, group=32,
                query_bits=0, key_format=0) -> Layout:
    return Layout(batch, n_q_heads, n_kv_heads, head_dim, k_bits, v_bits, group, capacity, query_bits,
                  key_format)


def bkv_cache_bytes(layout: Layout):
    a, b, c, d = C.c_size_t(), C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check("bkv_cache_bytes", _lib.bkv_cache_bytes(C.byref(layout), C.byref(a), C.byref(b), C.byref(c), C.byref(d)))
    return a.value, b.value, c.value, d.value


def bkv_k_meta_bytes(layout: Layout) -> int:
    out = C.c_size_t()
    _check("bkv_k_meta_bytes", _lib.bkv_k_meta_bytes(C.byref(layout), C.byref(out)))
    return out.value


def bkv_workspace_bytes(layout: Layout, max_len: int, k: int) -> int:
    out = C.c_size_t()
    _check("bkv_workspace_bytes", _lib.bkv_workspace_bytes(C.byref(layout), int(max_len), int(k), C.byref(out)))
    return out.value


@dataclass
class Cache:
    """torch-allocated buffers of one layer's cache plus the C view of them."""
    layout: Layout
    k_codes: object
    v_codes: object
    k_meta: object
    v_meta: object
    k_shadow: object
    v_shadow: object

    def view(self) -> CacheView:
        return CacheView(*(_ptr(getattr(self, n)) for n in ("k_codes", "v_codes", "k_meta", "v_meta",
                                                            "k_shadow", "v_shadow")))


def cache_rows(cache: Cache, b0: int, nb: int):
    """(layout, cache) of batch rows b0 .. b0 + nb - 1 of a cache: views of its
    buffers (every buffer is unit-major, unit = b * n_kv_heads + kvh), so
    calls on the slice read and write the same memory."""
    L = cache.layout
    units = L.batch * L.n_kv_heads
    lo, hi = b0 * L.n_kv_heads, (b0 + nb) * L.n_kv_heads
    part = lambda t: t[t.numel() // units * lo:t.numel() // units * hi]
    lay = make_layout(nb, L.n_q_heads, L.n_kv_heads, L.capacity, L.k_bits, L.v_bits, head_dim=L.head_dim,
                      group=L.group, query_bits=L.query_bits, key_format=L.key_format)
    return lay, Cache(lay, *(part(getattr(cache, n)) for n in ("k_codes", "v_codes", "k_meta", "v_meta",
                                                                 "k_shadow", "v_shadow")))


def allocate_cache(layout: Layout, device="cuda", shadow_on_host: bool = False) -> Cache:
    """Zero-filled cache buffers (torch).  With shadow_on_host the fp16 shadow
    rows live in pinned host memory that the GPU reads across PCIe."""
    import torch
    kb, vb, mb, sb = bkv_cache_bytes(layout)
    z8 = lambda n: torch.zeros(n, dtype=torch.uint8, device=device)
    z32 = lambda n: torch.zeros(n // 4, dtype=torch.int32, device=device)
    if shadow_on_host:
        sh = lambda n: torch.zeros(n // 2, dtype=torch.float16, pin_memory=True)
    else:
        sh = lambda n: torch.zeros(n // 2, dtype=torch.float16, device=device)
    return Cache(layout, z8(kb), z8(vb), z32(bkv_k_meta_bytes(layout)), z32(mb), sh(sb), sh(sb))


def kv_pack_append(layout: Layout, cache: Cache, k_new, v_new, n_new: int, pos_host, stream=None) -> None:
    pos = _host_i32(pos_host)
    view = cache.view()
    _check("kv_pack_append", _lib.kv_pack_append(C.byref(layout), C.byref(view), _ptr(k_new), _ptr(v_new),
                                                 int(n_new), pos.ctypes.data, _stream(stream)))


def qattn_decode_approx(layout: Layout, cache: Cache, q, len_host, sigma, ws, stream=None) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_decode_approx", _lib.qattn_decode_approx(C.byref(layout), C.byref(view), _ptr(q),
                                                           lens.ctypes.data, _ptr(sigma), _ptr(ws),
                                                           ws_bytes, _stream(stream)))


SELECT_AUTO, SELECT_IN_SCAN, SELECT_TWO_LAUNCHES = 0, 1, 2


def qattn_decode_select(layout: Layout, cache: Cache, q, len_host, k: int, sigma, idx, ws, stream=None,
                        mode: int = SELECT_AUTO) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_decode_select", _lib.qattn_decode_select(C.byref(layout), C.byref(view), _ptr(q),
                                                           lens.ctypes.data, int(k), _ptr(sigma), _ptr(idx),
                                                           _ptr(ws), ws_bytes, int(mode), _stream(stream)))


def qattn_decode_step(layout: Layout, cache: Cache, k_new, v_new, q, len_host, k: int, sigma, idx, ws, stream=None,
                      mode: int = SELECT_AUTO) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_decode_step", _lib.qattn_decode_step(C.byref(layout), C.byref(view), _ptr(k_new), _ptr(v_new),
                                                       _ptr(q), lens.ctypes.data, int(k), _ptr(sigma), _ptr(idx),
                                                       _ptr(ws), ws_bytes, int(mode), _stream(stream)))


def qattn_decode_fused(layout: Layout, cache: Cache, k_new, v_new, q, len_host, k: int, sigma, idx, out, ws,
                       stream=None) -> None:
    """The whole step in one launch; k_new = v_new = None: no append."""
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_decode_fused", _lib.qattn_decode_fused(C.byref(layout), C.byref(view), _ptr(k_new), _ptr(v_new),
                                                         _ptr(q), lens.ctypes.data, int(k), _ptr(sigma), _ptr(idx),
                                                         _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def bkv_fused_supported(layout: Layout, max_len: int, k: int) -> bool:
    out = C.c_int32()
    _check("bkv_fused_supported", _lib.bkv_fused_supported(C.byref(layout), int(max_len), int(k), C.byref(out)))
    return bool(out.value)


def bkv_select_in_scan(layout: Layout, max_len: int, k: int, mode: int = SELECT_AUTO) -> bool:
    out = C.c_int32()
    _check("bkv_select_in_scan", _lib.bkv_select_in_scan(C.byref(layout), int(max_len), int(k), int(mode),
                                                         C.byref(out)))
    return bool(out.value)


def topk_select(layout: Layout, sigma, len_host, k: int, idx, ws, stream=None) -> None:
    lens = _host_i32(len_host)
    ws_bytes = ws.numel() * ws.element_size()
    _check("topk_select", _lib.topk_select(C.byref(layout), _ptr(sigma), lens.ctypes.data, int(k), _ptr(idx),
                                           _ptr(ws), ws_bytes, _stream(stream)))


def topk_select_window(layout: Layout, sigma, len_host, k: int, window: int, idx, ws, stream=None) -> None:
    lens = _host_i32(len_host)
    ws_bytes = ws.numel() * ws.element_size()
    _check("topk_select_window", _lib.topk_select_window(C.byref(layout), _ptr(sigma), lens.ctypes.data, int(k),
                                                         int(window), _ptr(idx), _ptr(ws), ws_bytes,
                                                         _stream(stream)))


def topk_select_blocks(layout: Layout, sigma, len_host, n_blocks: int, block: int, idx, ws, stream=None) -> None:
    lens = _host_i32(len_host)
    ws_bytes = ws.numel() * ws.element_size()
    _check("topk_select_blocks", _lib.topk_select_blocks(C.byref(layout), _ptr(sigma), lens.ctypes.data,
                                                         int(n_blocks), int(block), _ptr(idx), _ptr(ws), ws_bytes,
                                                         _stream(stream)))


def qattn_correct(layout: Layout, cache: Cache, q, len_host, idx, k: int, ws, out, stream=None) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_correct", _lib.qattn_correct(C.byref(layout), C.byref(view), _ptr(q), lens.ctypes.data,
                                               _ptr(idx), int(k), _ptr(ws), ws_bytes, _ptr(out),
                                               _stream(stream)))


def qattn_score_select(layout: Layout, cache: Cache, q, len_host, k: int, sigma, idx, ws, stream=None,
                       mode: int = SELECT_AUTO) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_score_select", _lib.qattn_score_select(C.byref(layout), C.byref(view), _ptr(q), lens.ctypes.data,
                                                         int(k), _ptr(sigma), _ptr(idx), _ptr(ws), ws_bytes,
                                                         int(mode), _stream(stream)))


def qattn_decode_unselected(layout: Layout, cache: Cache, q, len_host, idx, k: int, ws, stream=None) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_decode_unselected", _lib.qattn_decode_unselected(C.byref(layout), C.byref(view), _ptr(q),
                                                                   lens.ctypes.data, _ptr(idx), int(k), _ptr(ws),
                                                                   ws_bytes, _stream(stream)))


def qattn_correct_unselected(layout: Layout, cache: Cache, q, len_host, idx, k: int, ws, out, stream=None) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_correct_unselected", _lib.qattn_correct_unselected(C.byref(layout), C.byref(view), _ptr(q),
                                                                     lens.ctypes.data, _ptr(idx), int(k),
                                                                     _ptr(ws), ws_bytes, _ptr(out),
                                                                     _stream(stream)))


def qattn_correct_hybrid(layout: Layout, cache: Cache, q, len_host, idx, k: int, exact_state, ws, out,
                         stream=None) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_correct_hybrid", _lib.qattn_correct_hybrid(C.byref(layout), C.byref(view), _ptr(q),
                                                             lens.ctypes.data, _ptr(idx), int(k), _ptr(exact_state),
                                                             _ptr(ws), ws_bytes, _ptr(out), _stream(stream)))


def qattn_exact_host(layout: Layout, k_shadow_host, v_shadow_host, q_host, len_host, idx_host, k: int, state_host,
                     n_threads: int = 0) -> None:
    """Host computation: every array argument is host memory (CPU tensors or
    numpy arrays)."""
    lens = _host_i32(len_host)
    _check("qattn_exact_host", _lib.qattn_exact_host(C.byref(layout), _hptr(k_shadow_host), _hptr(v_shadow_host),
                                                     _hptr(q_host), lens.ctypes.data, _hptr(idx_host), int(k),
                                                     _hptr(state_host), int(n_threads)))


def _hptr(a):
    """Address of a host array (torch CPU tensor or numpy array)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    assert not a.is_cuda, "host array expected"
    return a.data_ptr()


def raw_status(fn: str, *args) -> int:
    """Call an entry point with raw ctypes arguments and return its status
    (used to exercise the host-side error paths)."""
    return int(getattr(_lib, fn)(*args))


def qattn_decode_fused_noalloc(layout: Layout, cache: Cache, k_new, v_new, q, len_host, k: int, sigma, idx, out,
                               stream=None) -> None:
    """qattn_decode_fused on the library's own per-device workspace (no
    workspace argument; the call allocates nothing)."""
    lens = _host_i32(len_host)
    view = cache.view()
    _check("qattn_decode_fused_noalloc",
           _lib.qattn_decode_fused_noalloc(C.byref(layout), C.byref(view), _ptr(k_new), _ptr(v_new), _ptr(q),
                                           lens.ctypes.data, int(k), _ptr(sigma), _ptr(idx), _ptr(out),
                                           _stream(stream)))


def qattn_correct_blocks(layout: Layout, cache: Cache, q, len_host, idx, n_blocks: int, block: int, ws, out,
                         stream=None) -> None:
    lens = _host_i32(len_host)
    view = cache.view()
    ws_bytes = ws.numel() * ws.element_size()
    _check("qattn_correct_blocks", _lib.qattn_correct_blocks(C.byref(layout), C.byref(view), _ptr(q),
                                                             lens.ctypes.data, _ptr(idx), int(n_blocks), int(block),
                                                             _ptr(ws), ws_bytes, _ptr(out), _stream(stream)))


def qattn_hybrid_layers(layout: Layout, caches, qs, k_news, v_news, pos_host, k: int, micro: int, slots, outs,
                        n_threads: int = 0, stream=None) -> None:
    """caches, qs, k_news, v_news, outs: one per layer; slots: one dict per
    micro-batch with the HybridSlot fields (torch tensors; ws_bytes taken
    from ws)."""
    n = len(caches)
    views = (CacheView * n)(*(c.view() for c in caches))
    arr = lambda ts: (C.c_void_p * n)(*(_ptr(t) for t in ts))
    sl = (HybridSlot * len(slots))(*(HybridSlot(_ptr(d["sigma"]), _ptr(d["idx"]), _ptr(d["ws"]),
                                                d["ws"].numel() * d["ws"].element_size(), _ptr(d["state_dev"]),
                                                _ptr(d["idx_host"]), _ptr(d["q_host"]), _ptr(d["state_host"]))
                                     for d in slots))
    pos = _host_i32(pos_host)
    _check("qattn_hybrid_layers", _lib.qattn_hybrid_layers(C.byref(layout), n, views, arr(qs), arr(k_news),
                                                           arr(v_news), pos.ctypes.data, int(k), int(micro), sl,
                                                           arr(outs), int(n_threads), _stream(stream)))

