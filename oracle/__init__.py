"""CPU oracle for approximate-then-correct low-bit KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``bit_kv_attention_amd``) never imports it and shares no code with it.

The arithmetic lives in ``bitkv_oracle.c`` (plain C, scalar loops): the codec in
IEEE fp32, everything after it in fp64.  This module only builds that file with
gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitkv_oracle.c")
# BKV_SANITIZE=1: the same source under clang's AddressSanitizer and
# UndefinedBehaviorSanitizer (CPU checks; the sanitizer runtime must be
# preloaded, e.g. LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so))
_SANITIZE = os.environ.get("BKV_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE fp32: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        if _SANITIZE:
            cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fopenmp=libgomp", "-ffp-contract=off",
                   "-fno-fast-math", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-shared-libsan",
                   "-fPIC", "-shared", _SRC, "-o", tmp, "-lm", "-lgomp"]
        else:
            cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                   "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("B", "Hq", "Hkv", "D", "kbits", "vbits", "group", "cap", "kfmt")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        L.orc_f16_to_f32.argtypes = [C.c_uint16]
        L.orc_f16_to_f32.restype = C.c_float
        L.orc_f32_to_f16.argtypes = [C.c_float]
        L.orc_f32_to_f16.restype = C.c_uint16
        L.orc_quantize_rows.argtypes = [P, C.c_int, C.c_int, C.c_int, C.c_int, P, P]
        L.orc_k_bitpos.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int]
        L.orc_k_bitpos.restype = C.c_uint64
        L.orc_v_bitpos.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int]
        L.orc_v_bitpos.restype = C.c_uint64
        L.orc_get_bits.argtypes = [P, C.c_uint64, C.c_int]
        L.orc_get_bits.restype = C.c_uint32
        for f in ("orc_k_codes_bytes", "orc_v_codes_bytes", "orc_meta_bytes", "orc_k_meta_bytes",
                  "orc_shadow_bytes"):
            getattr(L, f).argtypes = [C.POINTER(_Shape)]
            getattr(L, f).restype = C.c_size_t
        L.orc_pack_append.argtypes = [C.POINTER(_Shape), P, P, P, P, P, P, P, P, C.c_int, P]
        L.orc_decode.argtypes = [C.POINTER(_Shape), P, P, P, P, P, P, P, P, C.c_int, P, P, P, P, P, P]
        L.orc_decode_q.argtypes = [C.POINTER(_Shape), P, P, P, P, P, P, P, P, C.c_int, P, C.c_int,
                                   P, P, P, P, P]
        L.orc_quantize_query.argtypes = [P, C.c_int, C.c_int, P, P]
        L.orc_quantize_group_mx.argtypes = [P, C.c_int, P, P]
        L.orc_quantize_block_mx8.argtypes = [P, C.c_int, P, P]
        L.orc_k_bitpos_mx8.argtypes = [C.c_int, C.c_int, C.c_int]
        L.orc_k_bitpos_mx8.restype = C.c_uint64
        L.orc_e2m1_value.argtypes = [C.c_uint32]
        L.orc_e2m1_value.restype = C.c_double
        L.orc_topk.argtypes = [P, C.c_int, C.c_int, P]
        L.orc_topk_window.argtypes = [P, C.c_int, C.c_int, C.c_int, P]
        L.orc_topk_blocks.argtypes = [P, C.c_int, C.c_int, C.c_int, P]
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_get_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


# ----------------------------------------------------------------- scalars

def f16_to_f32(bits: int) -> float:
    return float(lib().orc_f16_to_f32(int(bits)))


def f32_to_f16(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(np.float32(x))))


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


# ------------------------------------------------------------------- codec

def quantize_rows(x16: np.ndarray, group: int, bits: int):
    """O1 on rows of fp16 values.  x16: [..., D] float16.
    Returns (codes uint8 [..., D], scale16 uint16 [..., D/g], zero16 uint16 [..., D/g])."""
    x16 = np.ascontiguousarray(x16, dtype=np.float16)
    D = x16.shape[-1]
    n = int(np.prod(x16.shape[:-1])) if x16.ndim > 1 else 1
    codes = np.zeros(x16.shape, dtype=np.uint8)
    meta = np.zeros(x16.shape[:-1] + (D // group,), dtype=np.uint32)
    lib().orc_quantize_rows(_p(x16.view(np.uint16)), n, D, group, bits, _p(codes), _p(meta))
    return codes, (meta & 0xFFFF).astype(np.uint16), (meta >> 16).astype(np.uint16)


def quantize_rows_mx(x16: np.ndarray, group: int):
    """O1mx on rows of fp16 values.  x16: [..., D] float16.
    Returns (codes uint8 [..., D] = sign << 3 | E2M1 index, scale16 uint16 [..., D/g])."""
    x16 = np.ascontiguousarray(x16, dtype=np.float16)
    D = x16.shape[-1]
    rows = x16.reshape(-1, D)
    codes = np.zeros(rows.shape, dtype=np.uint8)
    sc = np.zeros((rows.shape[0], D // group), dtype=np.uint16)
    for r in range(rows.shape[0]):
        for p in range(D // group):
            seg = np.ascontiguousarray(rows[r, p * group:(p + 1) * group])
            cs = np.zeros(group, dtype=np.uint8)
            s16 = np.zeros(1, dtype=np.uint16)
            lib().orc_quantize_group_mx(_p(seg.view(np.uint16)), group, _p(cs), _p(s16))
            codes[r, p * group:(p + 1) * group] = cs
            sc[r, p] = s16[0]
    return codes.reshape(x16.shape), sc.reshape(x16.shape[:-1] + (D // group,))


def quantize_rows_mx8(x16: np.ndarray):
    """O1mx8 on rows of fp16 values, blocks of 32 channels.  x16: [..., D] float16.
    Returns (codes uint8 [..., D] = sign << 3 | E2M1 index, e8 uint8 [..., D/32]
    = X + 127, the block's scale being 2^X)."""
    x16 = np.ascontiguousarray(x16, dtype=np.float16)
    D = x16.shape[-1]
    rows = x16.reshape(-1, D)
    codes = np.zeros(rows.shape, dtype=np.uint8)
    e8 = np.zeros((rows.shape[0], D // 32), dtype=np.uint8)
    for r in range(rows.shape[0]):
        for p in range(D // 32):
            seg = np.ascontiguousarray(rows[r, p * 32:(p + 1) * 32])
            cs = np.zeros(32, dtype=np.uint8)
            e = np.zeros(1, dtype=np.uint8)
            lib().orc_quantize_block_mx8(_p(seg.view(np.uint16)), 32, _p(cs), _p(e))
            codes[r, p * 32:(p + 1) * 32] = cs
            e8[r, p] = e[0]
    return codes.reshape(x16.shape), e8.reshape(x16.shape[:-1] + (D // 32,))


def e2m1_value(code: int) -> float:
    return float(lib().orc_e2m1_value(int(code)))


def quantize_query(q16: np.ndarray, group: int):
    """O1q on one query row.  q16: [D] float16.
    Returns (codes int8 [D], scales float32 [D/group])."""
    q16 = np.ascontiguousarray(q16, dtype=np.float16).reshape(-1)
    D = q16.shape[0]
    codes = np.zeros(D, dtype=np.int8)
    scales = np.zeros(D // group, dtype=np.float32)
    lib().orc_quantize_query(_p(q16.view(np.uint16)), D, group, _p(codes), _p(scales))
    return codes, scales


def k_bitpos(t: int, c: int, D: int, bits: int) -> int:
    return int(lib().orc_k_bitpos(t, c, D, bits))


def k_bitpos_mx8(t: int, c: int, D: int) -> int:
    return int(lib().orc_k_bitpos_mx8(t, c, D))


def v_bitpos(t: int, c: int, D: int, bits: int) -> int:
    return int(lib().orc_v_bitpos(t, c, D, bits))


def get_bits(buf: np.ndarray, bitpos: int, nbits: int) -> int:
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    return int(lib().orc_get_bits(_p(buf), bitpos, nbits))


# ------------------------------------------------------------------- cache

@dataclass
class Shape:
    B: int
    Hq: int
    Hkv: int
    D: int
    kbits: int
    vbits: int
    group: int
    cap: int
    kfmt: int = 0  # keys: 0 affine codes; 1 MXFP4, fp16 query; 2 MXFP4 (E8M0 scales), FP4 query

    def c(self) -> _Shape:
        return _Shape(self.B, self.Hq, self.Hkv, self.D, self.kbits, self.vbits, self.group, self.cap, self.kfmt)


class Cache:
    """Host buffers of one layer's cache in the library's layout (see the C header)."""

    def __init__(self, s: Shape):
        self.s = s
        cs = s.c()
        L = lib()
        self.k_codes = np.zeros(L.orc_k_codes_bytes(C.byref(cs)), dtype=np.uint8)
        self.v_codes = np.zeros(L.orc_v_codes_bytes(C.byref(cs)), dtype=np.uint8)
        self.k_meta = np.zeros((L.orc_k_meta_bytes(C.byref(cs)) + 3) // 4, dtype=np.uint32)
        self.v_meta = np.zeros(L.orc_meta_bytes(C.byref(cs)) // 4, dtype=np.uint32)
        nsh = L.orc_shadow_bytes(C.byref(cs)) // 2
        self.k_shadow = np.zeros(nsh, dtype=np.uint16)
        self.v_shadow = np.zeros(nsh, dtype=np.uint16)

    def append(self, k_new: np.ndarray, v_new: np.ndarray, pos) -> None:
        """O1+O2.  k_new, v_new: [B][Hkv][n][D] float16; pos: [B] int."""
        s = self.s
        k_new = np.ascontiguousarray(k_new, dtype=np.float16)
        v_new = np.ascontiguousarray(v_new, dtype=np.float16)
        assert k_new.shape[:2] == (s.B, s.Hkv) and k_new.shape[3] == s.D
        n = k_new.shape[2]
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        assert np.all(pos + n <= s.cap)
        cs = s.c()
        lib().orc_pack_append(C.byref(cs), _p(self.k_codes), _p(self.v_codes), _p(self.k_meta),
                              _p(self.v_meta), _p(self.k_shadow), _p(self.v_shadow),
                              _p(k_new.view(np.uint16)), _p(v_new.view(np.uint16)), n, _p(pos))

    def decode(self, q: np.ndarray, lens, k: int, sel=None, want_approx=False, want_exact=False,
               qbits: int = 0):
        """O3..O5.  q: [B][Hq][D] float16.  qbits = 8: approximate logits against
        the INT8 query (O1q).  Returns dict(sigma, idx, out[, out_approx, out_exact])."""
        s = self.s
        q = np.ascontiguousarray(q, dtype=np.float16)
        assert q.shape == (s.B, s.Hq, s.D)
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        sigma = np.full((s.B, s.Hkv, s.cap), np.nan, dtype=np.float64)
        idx = np.full((s.B, s.Hkv, max(k, 0)), -1, dtype=np.int32)
        out = np.zeros((s.B, s.Hq, s.D), dtype=np.float64)
        oa = np.zeros_like(out) if want_approx else None
        oe = np.zeros_like(out) if want_exact else None
        sel_arr = None
        if sel is not None:
            sel_arr = np.ascontiguousarray(sel, dtype=np.int32)
            assert sel_arr.shape == (s.B, s.Hkv, k)
        cs = s.c()
        lib().orc_decode_q(C.byref(cs), _p(self.k_codes), _p(self.v_codes), _p(self.k_meta),
                           _p(self.v_meta), _p(self.k_shadow), _p(self.v_shadow),
                           _p(q.view(np.uint16)), _p(lens), int(k), _p(sel_arr), int(qbits),
                           _p(sigma), _p(idx), _p(out), _p(oa), _p(oe))
        r = {"sigma": sigma, "idx": idx, "out": out}
        if want_approx:
            r["out_approx"] = oa
        if want_exact:
            r["out_exact"] = oe
        return r

    # views used by tests
    def k_meta_planes(self):
        s = self.s
        return self.k_meta.reshape(s.B, s.Hkv, s.D // s.group, s.cap)

    def k_scales_e8(self):
        """Key format 2: the E8M0 bytes [B][Hkv][cap][D/32]."""
        s = self.s
        n = s.B * s.Hkv * s.cap * (s.D // 32)
        return self.k_meta.view(np.uint8)[:n].reshape(s.B, s.Hkv, s.cap, s.D // 32)

    def v_meta_planes(self):
        s = self.s
        return self.v_meta.reshape(s.B, s.Hkv, s.D // s.group, s.cap)


def topk(sigma: np.ndarray, k: int) -> np.ndarray:
    sigma = np.ascontiguousarray(sigma, dtype=np.float64)
    idx = np.full(max(k, 0), -1, dtype=np.int32)
    lib().orc_topk(_p(sigma), int(sigma.shape[0]), int(k), _p(idx))
    return idx


def topk_window(sigma: np.ndarray, k: int, w: int) -> np.ndarray:
    """O4 with the last w tokens always selected (k + w slots, see the C header)."""
    sigma = np.ascontiguousarray(sigma, dtype=np.float64)
    idx = np.full(max(k + w, 0), -1, dtype=np.int32)
    lib().orc_topk_window(_p(sigma), int(sigma.shape[0]), int(k), int(w), _p(idx))
    return idx


def topk_blocks(sigma: np.ndarray, nb: int, bs: int) -> np.ndarray:
    """O4 by blocks of bs tokens scored by their largest sigma (nb * bs slots,
    see the C header)."""
    sigma = np.ascontiguousarray(sigma, dtype=np.float64)
    idx = np.full(max(nb * bs, 0), -1, dtype=np.int32)
    lib().orc_topk_blocks(_p(sigma), int(sigma.shape[0]), int(nb), int(bs), _p(idx))
    return idx
