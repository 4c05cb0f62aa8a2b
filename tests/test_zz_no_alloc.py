"""qattn_decode_fused_noalloc: the fused step on the library's own per-device
workspace (for callers that cannot allocate).  Checked against
qattn_decode_fused with a caller workspace on the same inputs, over two calls
in a row, the second with fewer (batch, KV head) pairs and shorter lengths,
so the array starts each call from what the previous call left; and its
host-side argument errors."""
import ctypes as C

import numpy as np
import pytest

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_noalloc_host_errors():
    from bit_kv_attention_amd import binding as bk
    fn = "qattn_decode_fused_noalloc"
    lay = bk.make_layout(4, 32, 8, 1024, 4, 4)
    cv = bk.CacheView(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    lens = np.full(4, 100, np.int32)
    P = lens.ctypes.data
    pre = (C.byref(lay), C.byref(cv))
    assert bk.raw_status(fn, *pre, FAKE, None, FAKE, P, 8, FAKE, FAKE, FAKE, None) == 1  # one of k_new, v_new
    assert bk.raw_status(fn, *pre, FAKE, FAKE, FAKE, P, -1, FAKE, FAKE, FAKE, None) == 7
    assert bk.raw_status(fn, *pre, FAKE, FAKE, FAKE, P, 8, FAKE, None, FAKE, None) == 1
    assert bk.raw_status(fn, *pre, FAKE, FAKE, None, P, 8, FAKE, FAKE, FAKE, None) == 1
    zero = np.array([100, 0, 5, 5], np.int32)  # an append needs len >= 1
    assert bk.raw_status(fn, *pre, FAKE, FAKE, FAKE, zero.ctypes.data, 8, FAKE, FAKE, FAKE, None) == 4
    bad = bk.CacheView(FAKE, None, FAKE, FAKE, FAKE, FAKE)
    assert bk.raw_status(fn, C.byref(lay), C.byref(bad), FAKE, FAKE, FAKE, P, 8, FAKE, FAKE, FAKE, None) == 1
    # more workspace than the library's 64 MiB array: refused before any launch
    big = bk.make_layout(4, 8, 2, 1 << 20, 4, 4)
    bl = np.full(4, 1 << 20, np.int32)
    assert bk.bkv_workspace_bytes(big, 1 << 20, 100000) > 64 << 20
    assert bk.raw_status(fn, C.byref(big), C.byref(cv), FAKE, FAKE, FAKE, bl.ctypes.data, 100000, FAKE, FAKE,
                         FAKE, None) == 5
    # a layout the fused step does not take (the INT8 query): refused by the
    # host-side shape check, before any device call -- every call here must
    # fail on the host, since the pointers are fake (key format 2, taken by
    # the fused step, would launch on them where a GPU is present)
    q8 = bk.make_layout(4, 32, 8, 1024, 4, 4, query_bits=8)
    assert bk.raw_status(fn, C.byref(q8), C.byref(cv), FAKE, FAKE, FAKE, P, 8, FAKE, FAKE, FAKE, None) == 3


@pytest.mark.gpu
def test_noalloc_matches_fused_with_workspace(orc):
    import torch
    import parity as Pm
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    calls = [
        (Pm.Workload("na1", 4, 32, 8, 128, 9000, 4, 4, 32, 128, 16, 901), np.array([9000, 8191, 4000, 77])),
        (Pm.Workload("na2", 2, 16, 2, 128, 3000, 3, 2, 32, 64, 8, 902), np.array([2999, 1234])),
    ]
    for i, (w, lens) in enumerate(calls):
        print(f"\n[case] no-alloc call {i}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} L={w.L} k={w.k} "
              f"kb={w.kbits} vb={w.vbits}", flush=True)
        pair = Pm.build_pair(w, L=w.L)
        lay, cap = pair["lay"], pair["cap"]
        assert bk.bkv_fused_supported(lay, int(lens.max()), w.k)
        gc2 = bk.allocate_cache(lay)
        for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow"):
            getattr(gc2, name).copy_(getattr(pair["gc"], name))
        pos = [int(x) - 1 for x in lens]
        q, kn, vn = Pm.to_dev(pair["q"]), Pm.to_dev(pair["k1"]), Pm.to_dev(pair["v1"])
        ref = DecodeStep(lay, w.k, int(lens.max()), one_launch=True)
        assert ref.one_launch
        ref.step(pair["gc"], q, kn, vn, pos)
        dev = torch.device("cuda:0")
        sigma = torch.full((w.B * w.Hkv * cap,), float("nan"), dtype=torch.float32, device=dev)
        idx = torch.full((w.B * w.Hkv * w.k,), -7, dtype=torch.int32, device=dev)
        out = torch.full((w.B * w.Hq * 128,), float("nan"), dtype=torch.float32, device=dev)
        bk.qattn_decode_fused_noalloc(lay, gc2, kn, vn, q, lens, w.k, sigma, idx, out)
        torch.cuda.synchronize()
        print(f"[case] no-alloc call {i} ran", flush=True)
        for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow"):
            assert torch.equal(getattr(gc2, name), getattr(pair["gc"], name)), name
        a_sig = ref.sigma.cpu().numpy().reshape(w.B, w.Hkv, cap)
        b_sig = sigma.cpu().numpy().reshape(w.B, w.Hkv, cap)
        for b in range(w.B):
            assert np.array_equal(a_sig[b, :, :lens[b]], b_sig[b, :, :lens[b]]), (i, b)
        assert np.array_equal(ref.idx.cpu().numpy().reshape(-1)[:w.B * w.Hkv * w.k], idx.cpu().numpy()), i
        Pm.assert_close(out.cpu().numpy(), ref.out.cpu().numpy().reshape(-1), f"call {i} out vs fused")
        # and against the oracle on the selected set
        pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
        sel = idx.cpu().numpy().reshape(w.B, w.Hkv, w.k)
        orc = pair["oc"].decode(pair["q"], lens, w.k, sel=sel)
        Pm.assert_close(out.cpu().numpy().reshape(w.B, w.Hq, 128), orc["out"], f"call {i} out vs oracle(S_gpu)")
