"""The C-ABI library loads, exports every entry point include/bitkv.h declares,
and rejects bad arguments on the host before any launch (no GPU needed); the
one host-only computation (qattn_exact_host) against fp64."""
import ctypes as C
import os
import re

import numpy as np

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bk():
    lib = os.path.join(ROOT, "bit_kv_attention_amd", "libbitkv.so")
    if not os.path.exists(lib):
        from bit_kv_attention_amd import build as b
        b.build()
    import bit_kv_attention_amd.binding as bk
    return bk


def declared_functions():
    with open(os.path.join(ROOT, "include", "bitkv.h")) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", txt, flags=re.M)))


def test_every_declared_symbol_is_exported(bk):
    names = declared_functions()
    assert set(names) == set(bk.EXPORTED), names
    for n in names:
        assert hasattr(bk._lib, n), n


def L(bk, **kw):
    a = dict(batch=4, n_q_heads=32, n_kv_heads=8, capacity=1024, k_bits=4, v_bits=4)
    a.update(kw)
    return bk.make_layout(**a)


def test_cache_and_workspace_sizes(bk):
    kb, vb, mb, sb = bk.bkv_cache_bytes(L(bk, k_bits=3, v_bits=2))
    units = 32
    assert kb == units * 1024 * 48
    assert vb == units * 1024 * 32
    assert mb == units * 4 * 1024 * 4
    assert sb == units * 1024 * 128 * 2
    kb2, _, mb64, _ = bk.bkv_cache_bytes(L(bk, k_bits=2, group=64))  # 2-bit keys; one meta word per 64 channels
    assert kb2 == units * 1024 * 128 * 2 // 8 and mb64 == units * 2 * 1024 * 4
    # key meta: the planes for key formats 0 and 1, one word of four E8M0 bytes per token for format 2
    assert bk.bkv_k_meta_bytes(L(bk, k_bits=3, v_bits=2)) == mb
    assert bk.bkv_k_meta_bytes(L(bk, k_bits=4, key_format=1)) == mb
    assert bk.bkv_k_meta_bytes(L(bk, k_bits=4, key_format=2)) == units * 1024 * 4
    w1 = bk.bkv_workspace_bytes(L(bk), 1024, 64)
    w0 = bk.bkv_workspace_bytes(L(bk), 0, 0)
    assert w1 >= 4 * 32 * 130 * 4 + 4 * 32 * 2 * 260 * 4 and w0 > 0
    # the bound covers every shorter step
    for m in range(0, 1025, 37):
        assert bk.bkv_workspace_bytes(L(bk), m, 64) <= w1


@pytest.mark.parametrize("kw,status", [
    (dict(k_bits=5), 3), (dict(v_bits=3), 3), (dict(n_q_heads=30), 2), (dict(n_q_heads=16, n_kv_heads=16), 3),
    (dict(capacity=1000), 2), (dict(capacity=0), 2), (dict(batch=257), 3), (dict(batch=0), 2),
])
def test_bad_layouts_rejected(bk, kw, status):
    a, b, c, d = C.c_size_t(), C.c_size_t(), C.c_size_t(), C.c_size_t()
    lay = L(bk, **kw)
    assert bk.raw_status("bkv_cache_bytes", C.byref(lay), C.byref(a), C.byref(b), C.byref(c), C.byref(d)) == status


def test_unsupported_head_dim_and_group(bk):
    out = C.c_size_t()
    lay = bk.Layout(4, 32, 8, 64, 4, 4, 32, 1024)
    assert bk.raw_status("bkv_workspace_bytes", C.byref(lay), 10, 4, C.byref(out)) == 3
    lay = bk.Layout(4, 32, 8, 128, 4, 4, 16, 1024)  # groups of 32 and 64 channels only
    assert bk.raw_status("bkv_workspace_bytes", C.byref(lay), 10, 4, C.byref(out)) == 3
    lay = bk.Layout(4, 32, 8, 128, 4, 4, 128, 1024)
    assert bk.raw_status("bkv_workspace_bytes", C.byref(lay), 10, 4, C.byref(out)) == 3
    lay = bk.Layout(4, 32, 8, 128, 5, 4, 32, 1024)  # key bits 1..4
    assert bk.raw_status("bkv_workspace_bytes", C.byref(lay), 10, 4, C.byref(out)) == 3
    lay = bk.Layout(4, 32, 8, 128, 2, 4, 64, 1024)
    assert bk.raw_status("bkv_workspace_bytes", C.byref(lay), 10, 4, C.byref(out)) == 0
    for qb, want in ((8, 0), (4, 3), (16, 3), (-1, 3)):  # query of the approximate scores: fp16 or INT8
        lay = bk.Layout(4, 32, 8, 128, 4, 4, 32, 1024, qb)
        assert bk.raw_status("bkv_workspace_bytes", C.byref(lay), 10, 4, C.byref(out)) == want, qb
    # key formats 1 and 2 (MXFP4) need 4-bit keys, groups of 32 and query_bits 0
    for args, want in (((4, 32, 0, 1), 0), ((3, 32, 0, 1), 3), ((4, 64, 0, 1), 3), ((4, 32, 8, 1), 3),
                       ((4, 32, 0, 2), 0), ((3, 32, 0, 2), 3), ((4, 64, 0, 2), 3), ((4, 32, 8, 2), 3),
                       ((4, 32, 0, 3), 3), ((4, 32, 0, -1), 3)):
        kb, g, qb, kf = args
        lay = bk.Layout(4, 32, 8, 128, kb, 4, g, 1024, qb, kf)
        assert bk.raw_status("bkv_workspace_bytes", C.byref(lay), 10, 4, C.byref(out)) == want, args
    assert bk.raw_status("bkv_workspace_bytes", None, 10, 4, C.byref(out)) == 1
    lay = bk.Layout(4, 32, 8, 128, 4, 4, 32, 1024)
    assert bk.raw_status("bkv_workspace_bytes", C.byref(lay), 10, -1, C.byref(out)) == 7


def test_fused_supported_shapes(bk):
    """Which calls the one-launch step takes (host logic only): the fp16 query
    with 3- or 4-bit affine keys or 4-bit MXFP4 keys of both formats; not the
    INT8 query nor 1- and 2-bit keys; not more than 256 (b, kvh) pairs; not
    more splits times k than the lists hold."""
    def sup(*args, max_len=32768, k=256):
        return bk.bkv_fused_supported(bk.Layout(*args), max_len, k)
    assert sup(4, 32, 8, 128, 4, 4, 32, 32768)
    assert sup(4, 32, 8, 128, 3, 2, 32, 32768)
    assert sup(4, 64, 8, 128, 3, 2, 32, 131072, max_len=131072, k=512)
    assert sup(4, 32, 8, 128, 4, 4, 32, 32768, 0, 1)  # MXFP4 keys, fp16 query
    assert sup(4, 32, 8, 128, 4, 2, 32, 32768, 0, 2)  # MXFP4 keys and query
    assert not sup(4, 32, 8, 128, 4, 4, 32, 32768, 8)  # INT8 query
    assert not sup(4, 32, 8, 128, 2, 2, 64, 32768)
    assert not sup(4, 32, 8, 128, 1, 2, 64, 32768)
    assert not sup(64, 32, 8, 128, 4, 4, 32, 4096, max_len=4096)  # 512 (b, kvh) pairs
    assert sup(1, 4, 1, 128, 4, 4, 32, 4096, max_len=4096, k=100)
    assert not sup(1, 4, 1, 128, 4, 4, 32, 4096, max_len=4096, k=4096)  # splits x k over the lists' room


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def fake_cache(bk):
    return bk.CacheView(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def test_host_error_paths(bk):
    import numpy as np
    lay = L(bk)
    cv = fake_cache(bk)
    pos = np.zeros(4, np.int32)
    lens = np.full(4, 100, np.int32)
    P = lambda a: a.ctypes.data
    # NULL cache member
    bad = bk.CacheView(FAKE, None, FAKE, FAKE, FAKE, FAKE)
    assert bk.raw_status("kv_pack_append", C.byref(lay), C.byref(bad), FAKE, FAKE, 1, P(pos), None) == 1
    # capacity: pos + n_new > capacity, negative pos
    p2 = np.array([0, 0, 1024, 0], np.int32)
    assert bk.raw_status("kv_pack_append", C.byref(lay), C.byref(cv), FAKE, FAKE, 1, P(p2), None) == 4
    p3 = np.array([0, -1, 0, 0], np.int32)
    assert bk.raw_status("kv_pack_append", C.byref(lay), C.byref(cv), FAKE, FAKE, 1, P(p3), None) == 4
    assert bk.raw_status("kv_pack_append", C.byref(lay), C.byref(cv), FAKE, FAKE, -1, P(pos), None) == 7
    # n_new == 0 enqueues nothing and succeeds
    assert bk.raw_status("kv_pack_append", C.byref(lay), C.byref(cv), FAKE, FAKE, 0, P(pos), None) == 0
    # lengths beyond capacity
    l2 = np.array([100, 2000, 5, 5], np.int32)
    assert bk.raw_status("qattn_decode_approx", C.byref(lay), C.byref(cv), FAKE, P(l2), FAKE, FAKE,
                         1 << 30, None) == 4
    # workspace too small (64 bytes is below every region: no call below may
    # reach a launch, the pointers are fake)
    need = bk.bkv_workspace_bytes(lay, 100, 8)
    assert bk.raw_status("qattn_decode_approx", C.byref(lay), C.byref(cv), FAKE, P(lens), FAKE, FAKE,
                         64, None) == 5
    assert bk.raw_status("qattn_correct", C.byref(lay), C.byref(cv), FAKE, P(lens), FAKE, 8, FAKE,
                         64, FAKE, None) == 5
    # k < 0, NULL idx with k > 0, k == 0 is a no-op for top-k
    assert bk.raw_status("topk_select", C.byref(lay), FAKE, P(lens), -1, FAKE, FAKE, need, None) == 7
    assert bk.raw_status("topk_select", C.byref(lay), FAKE, P(lens), 4, None, FAKE, need, None) == 1
    assert bk.raw_status("topk_select", C.byref(lay), FAKE, P(lens), 4, FAKE, None, need, None) == 1
    assert bk.raw_status("topk_select", C.byref(lay), FAKE, P(lens), 4, FAKE, FAKE, 100, None) == 5
    assert bk.raw_status("topk_select", C.byref(lay), FAKE, P(lens), 0, None, None, 0, None) == 0
    assert bk.raw_status("qattn_correct", C.byref(lay), C.byref(cv), FAKE, P(lens), None, 4, FAKE,
                         need, FAKE, None) == 1
    assert bk.raw_status("qattn_correct", C.byref(lay), C.byref(cv), FAKE, P(lens), FAKE, -2, FAKE,
                         need, FAKE, None) == 7
    # NULL length array
    assert bk.raw_status("topk_select", C.byref(lay), FAKE, None, 4, FAKE, FAKE, need, None) == 1
    # the recent-window variant: negative or overflowing sizes, NULL idx, a
    # workspace sized for k alone (the row is k + window), the empty row
    tw = "topk_select_window"
    assert bk.raw_status(tw, C.byref(lay), FAKE, P(lens), 4, -1, FAKE, FAKE, need, None) == 7
    assert bk.raw_status(tw, C.byref(lay), FAKE, P(lens), -1, 4, FAKE, FAKE, need, None) == 7
    assert bk.raw_status(tw, C.byref(lay), FAKE, P(lens), 2**31 - 4, 8, FAKE, FAKE, need, None) == 7
    assert bk.raw_status(tw, C.byref(lay), FAKE, P(lens), 0, 4, None, FAKE, need, None) == 1
    assert bk.raw_status(tw, C.byref(lay), FAKE, P(lens), 4, 1000, FAKE, FAKE, need, None) == 5
    assert bk.raw_status(tw, C.byref(lay), FAKE, P(lens), 0, 0, None, None, 0, None) == 0
    assert bk.raw_status(tw, C.byref(lay), FAKE, P(l2), 4, 4, FAKE, FAKE, 1 << 30, None) == 4
    # the unselected-token pass and its merge; the in-launch selection
    for fn, extra in (("qattn_decode_unselected", ()), ("qattn_correct_unselected", (FAKE,))):
        pre = (C.byref(lay), C.byref(cv), FAKE, P(lens))
        assert bk.raw_status(fn, *pre, FAKE, -1, FAKE, need, *extra, None) == 7
        assert bk.raw_status(fn, *pre, None, 4, FAKE, need, *extra, None) == 1
        assert bk.raw_status(fn, *pre, FAKE, 4, FAKE, 64, *extra, None) == 5
        assert bk.raw_status(fn, C.byref(lay), C.byref(cv), FAKE, P(l2), FAKE, 4, FAKE, need, *extra, None) == 4
    ds = "qattn_decode_select"
    pre = (C.byref(lay), C.byref(cv), FAKE, P(lens))
    assert bk.raw_status(ds, *pre, -1, FAKE, FAKE, FAKE, need, 0, None) == 7
    assert bk.raw_status(ds, *pre, 4, FAKE, FAKE, FAKE, need, 3, None) == 7
    assert bk.raw_status(ds, *pre, 4, FAKE, None, FAKE, need, 0, None) == 1
    assert bk.raw_status(ds, *pre, 4, FAKE, FAKE, FAKE, 64, 0, None) == 5
    # block selection: block not a power of two in [32, 1024], negative or
    # overflowing budget, NULL idx, bad length, the empty budget
    tb = "topk_select_blocks"
    for blk in (0, 16, 48, 2048, -128):
        assert bk.raw_status(tb, C.byref(lay), FAKE, P(lens), 4, blk, FAKE, FAKE, need, None) == 7, blk
    assert bk.raw_status(tb, C.byref(lay), FAKE, P(lens), -1, 128, FAKE, FAKE, need, None) == 7
    assert bk.raw_status(tb, C.byref(lay), FAKE, P(lens), 2**24, 1024, FAKE, FAKE, need, None) == 7
    assert bk.raw_status(tb, C.byref(lay), FAKE, P(lens), 4, 128, None, FAKE, need, None) == 1
    assert bk.raw_status(tb, C.byref(lay), FAKE, P(lens), 4, 128, FAKE, None, need, None) == 1
    assert bk.raw_status(tb, C.byref(lay), FAKE, P(lens), 4, 128, FAKE, FAKE, 64, None) == 5
    assert bk.raw_status(tb, C.byref(lay), FAKE, P(l2), 4, 128, FAKE, FAKE, need, None) == 4
    assert bk.raw_status(tb, C.byref(lay), FAKE, P(lens), 0, 128, None, None, 0, None) == 0
    big = L(bk, capacity=32 * 8192 + 32)  # 8193 blocks of 32 tokens
    assert bk.raw_status(tb, C.byref(big), FAKE, P(lens), 4, 32, FAKE, FAKE, need, None) == 3


def test_hybrid_layers_host_errors(bk):
    """qattn_hybrid_layers validates everything before enqueueing anything
    (the pointers here are fake and never dereferenced)."""
    import numpy as np
    fn = "qattn_hybrid_layers"
    lay = L(bk)  # batch 4
    cv = (bk.CacheView * 2)(fake_cache(bk), fake_cache(bk))
    ptrs = (C.c_void_p * 2)(FAKE, FAKE)
    pos = np.full(4, 100, np.int32)
    need = bk.bkv_workspace_bytes(bk.make_layout(2, 32, 8, 1024, 4, 4), 101, 8)
    slot = lambda ws_bytes: bk.HybridSlot(FAKE, FAKE, FAKE, ws_bytes, FAKE, FAKE, FAKE, FAKE)
    slots = (bk.HybridSlot * 2)(slot(need), slot(need))
    P = pos.ctypes.data
    args = lambda **kw: [kw.get("lay", C.byref(lay)), kw.get("n", 2), kw.get("cv", cv), ptrs, ptrs, ptrs,
                         kw.get("pos", P), kw.get("k", 8), kw.get("micro", 2), kw.get("slots", slots), ptrs,
                         kw.get("threads", 0), None]
    assert bk.raw_status(fn, *args(micro=3)) == 7      # 4 rows do not split in 3
    assert bk.raw_status(fn, *args(micro=0)) == 7
    assert bk.raw_status(fn, *args(k=-1)) == 7
    assert bk.raw_status(fn, *args(threads=-1)) == 7
    assert bk.raw_status(fn, *args(n=0)) == 0           # nothing to do
    assert bk.raw_status(fn, *args(lay=None)) == 1
    bad = np.array([100, 1024, 5, 5], np.int32)        # a position at the capacity
    assert bk.raw_status(fn, *args(pos=bad.ctypes.data)) == 4
    small = (bk.HybridSlot * 2)(slot(need), slot(64))
    assert bk.raw_status(fn, *args(slots=small)) == 5
    nulls = (bk.HybridSlot * 2)(slot(need), bk.HybridSlot(FAKE, None, FAKE, need, FAKE, FAKE, FAKE, FAKE))
    assert bk.raw_status(fn, *args(slots=nulls)) == 1   # no idx with k > 0
    cv2 = (bk.CacheView * 2)(fake_cache(bk), bk.CacheView(FAKE, FAKE, FAKE, FAKE, None, FAKE))
    assert bk.raw_status(fn, *args(cv=cv2)) == 1


def test_status_strings(bk):
    for s in range(8):
        assert bk._lib.bkv_status_string(s)
    with pytest.raises(bk.BitKVError):
        bk.bkv_workspace_bytes(L(bk, k_bits=7), 5, 1)


def test_exact_host_state(bk):
    """qattn_exact_host (host code) against the exact state in fp64 on small
    inputs: ragged and empty sequences, -1 and out-of-range row entries, k
    past the length, both GQA groups; and its argument errors."""
    rng = np.random.default_rng(5)
    for G in (4, 8):
        B, Hkv, D, cap = 3, 2, 128, 96
        lay = L(bk, batch=B, n_q_heads=G * Hkv, n_kv_heads=Hkv, capacity=cap)
        K = (rng.standard_normal((B, Hkv, cap, D)) * 2).astype(np.float16)
        V = rng.standard_normal((B, Hkv, cap, D)).astype(np.float16)
        q = rng.standard_normal((B, G * Hkv, D)).astype(np.float16)
        lens = np.array([96, 41, 0], np.int32)
        k = 50
        idx = np.full((B, Hkv, k), -1, np.int32)
        for b in range(B):
            for h in range(Hkv):
                n = lens[b]
                sel = rng.choice(n, size=min(k - 5, n), replace=False) if n else np.array([], int)
                idx[b, h, :len(sel)] = np.sort(sel)
                if n:
                    idx[b, h, len(sel)] = n + 3  # outside [0, len): skipped
        state = np.zeros((B, G * Hkv, D + 2), np.float32)
        assert bk.qattn_exact_host(lay, K, V, q, lens, idx, k, state, 2) is None
        for b in range(B):
            for hq in range(G * Hkv):
                kvh = hq // G
                n = lens[b]
                ts = [t for t in idx[b, kvh, :min(k, n)] if 0 <= t < n]
                if not ts:
                    assert state[b, hq, 0] == -np.inf and state[b, hq, 1] == 0 and not state[b, hq, 2:].any()
                    continue
                lam = K[b, kvh, ts].astype(np.float64) @ q[b, hq].astype(np.float64) / np.sqrt(D) / np.log(2)
                m = lam.max()
                w = np.exp2(lam - m)
                np.testing.assert_allclose(state[b, hq, 0], m, rtol=1e-5, atol=1e-5)
                np.testing.assert_allclose(state[b, hq, 1], w.sum(), rtol=1e-4)
                np.testing.assert_allclose(state[b, hq, 2:], w @ V[b, kvh, ts].astype(np.float64), rtol=1e-4, atol=1e-4)
    ex = "qattn_exact_host"
    P = lambda a: a.ctypes.data_as(C.c_void_p)
    assert bk.raw_status(ex, C.byref(lay), P(K), P(V), P(q), P(lens), P(idx), -1, P(state), 1) == 7
    assert bk.raw_status(ex, C.byref(lay), P(K), P(V), P(q), P(lens), P(idx), 4, P(state), -1) == 7
    assert bk.raw_status(ex, C.byref(lay), None, P(V), P(q), P(lens), P(idx), 4, P(state), 1) == 1
    assert bk.raw_status(ex, C.byref(lay), P(K), P(V), P(q), P(lens), None, 4, P(state), 1) == 1
    bad = np.array([97, 0, 0], np.int32)
    assert bk.raw_status(ex, C.byref(lay), P(K), P(V), P(q), P(bad), P(idx), 4, P(state), 1) == 4
