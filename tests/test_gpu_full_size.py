"""GPU parity at the full sizes of the five decode-attention workloads and the
low-bit codec workloads (1- and 2-bit keys, the INT8 query, MXFP4 keys), in the launch configuration the benchmark times:
the whole batch runs on the GPU; the oracle recomputes sampled (batch, KV head)
units one by one."""
import numpy as np
import pytest

from bit_kv_attention_amd.synth import CODEC_WORKLOADS, WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P(orc):
    import parity
    return parity


def unit_slices(arr, units):
    return arr.reshape(units, -1)


@pytest.mark.parametrize("name", [w.name for w in WORKLOADS + CODEC_WORKLOADS])
def test_full_size_sampled_units(P, name):
    import torch
    import oracle
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    from bit_kv_attention_amd.synth import BY_NAME, make_inputs, make_new_tokens
    w = BY_NAME[name]
    print(f"\n[case] full size {w.name}", flush=True)
    L = w.L
    cap = ((L + 31) // 32) * 32
    inp = make_inputs(w, L=L - 1)
    kn, vn = make_new_tokens(w, 1, inp.outlier_ch)
    lay = bk.make_layout(w.B, w.Hq, w.Hkv, cap, w.kbits, w.vbits, group=w.group, query_bits=w.query_bits,
                         key_format=w.key_format)
    gc = bk.allocate_cache(lay)
    bk.kv_pack_append(lay, gc, P.to_dev(inp.K), P.to_dev(inp.V), L - 1, [0] * w.B)
    st = DecodeStep(lay, w.k, L)
    out = st.step(gc, P.to_dev(inp.q), P.to_dev(kn[0]), P.to_dev(vn[0]), [L - 1] * w.B)
    torch.cuda.synchronize()
    units = w.B * w.Hkv
    g_out = out.cpu().numpy().reshape(w.B, w.Hq, 128)
    g_sig = st.sigma.cpu().numpy().reshape(units, cap)
    g_idx = st.idx.cpu().numpy().reshape(units, w.k)
    g_buf = {n: unit_slices(getattr(gc, n).cpu().numpy().view(np.uint8), units)
             for n in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow")}
    for u in sorted({0, units - 1}):
        b, h = divmod(u, w.Hkv)
        print(f"[case] {w.name} unit {u}", flush=True)
        oc = oracle.Cache(oracle.Shape(1, w.G, 1, 128, w.kbits, w.vbits, w.group, cap, w.key_format))
        oc.append(inp.K[b:b + 1, h:h + 1], inp.V[b:b + 1, h:h + 1], np.zeros(1, np.int32))
        oc.append(kn[0][b:b + 1, h:h + 1], vn[0][b:b + 1, h:h + 1], np.array([L - 1], np.int32))
        for name, ob in P.orc_buffers(oc).items():
            assert np.array_equal(g_buf[name][u], ob), (name, u)
        q = np.ascontiguousarray(inp.q[b:b + 1, h * w.G:(h + 1) * w.G])
        ref = oc.decode(q, np.array([L], np.int32), w.k, qbits=w.query_bits)
        np.testing.assert_allclose(g_sig[u, :L], ref["sigma"][0, 0, :L], rtol=1e-5, atol=2e-5)
        assert np.array_equal(g_idx[u], oracle.topk(g_sig[u, :L].astype(np.float64), w.k))
        P.assert_topk_near_tie(g_idx[u], ref["idx"][0, 0], ref["sigma"][0, 0], L, f"unit {u}")
        if w.planted and w.kbits >= 3:  # (1- and 2-bit keys may rank a planted token lower)
            assert set(inp.planted_pos[b, h].tolist()) <= set(g_idx[u].tolist())
        ref_s = oc.decode(q, np.array([L], np.int32), w.k, sel=g_idx[u].reshape(1, 1, -1), qbits=w.query_bits)
        P.assert_close(g_out[b, h * w.G:(h + 1) * w.G], ref_s["out"][0], f"unit {u} vs oracle(S_gpu)")
        P.assert_close(g_out[b, h * w.G:(h + 1) * w.G], ref["out"][0], f"unit {u} vs oracle(S_oracle)")
