"""GPU parity at the full sizes of the five decode-attention workloads and the
low-bit codec workloads (1- and 2-bit keys, the INT8 query, MXFP4 keys), in the
launch configurations the benchmark times: the whole batch runs on the GPU,
through the fused launch and through the separate launches where the layout
has both; the oracle recomputes (batch, KV head) units stacked as the KV
heads of one oracle batch row -- every unit of the 32K workloads, eight
spread over the batch at 128K.  Each case prints its worst output error as a
fraction of the tolerance (the margin of the subtraction form).
The 70B workload also runs with its shadow rows in pinned host memory (the
correction then gathers them across PCIe)."""
import numpy as np
import pytest

from bit_kv_attention_amd.synth import CODEC_WORKLOADS, WORKLOADS

pytestmark = pytest.mark.gpu

CASES = [(w.name, "hbm") for w in WORKLOADS + CODEC_WORKLOADS] + [("llama70b_k3v2_L131072", "host")]


@pytest.fixture(scope="module")
def P(orc):
    import parity
    return parity


def unit_slices(arr, units):
    return arr.reshape(units, -1)


@pytest.mark.parametrize("name,shadow", CASES)
def test_full_size_sampled_units(P, name, shadow):
    import torch
    import oracle
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    from bit_kv_attention_amd.synth import BY_NAME, make_inputs, make_new_tokens
    w = BY_NAME[name]
    print(f"\n[case] full size {w.name}, shadow in {shadow}", flush=True)
    L = w.L
    cap = ((L + 31) // 32) * 32
    units = w.B * w.Hkv
    sample = list(range(units)) if L <= 32768 else sorted({(j * (units - 1)) // 7 for j in range(8)})
    inp = make_inputs(w, L=L - 1)
    kn, vn = make_new_tokens(w, 1, inp.outlier_ch)
    lay = bk.make_layout(w.B, w.Hq, w.Hkv, cap, w.kbits, w.vbits, group=w.group, query_bits=w.query_bits,
                         key_format=w.key_format)
    fused_ok = (not (w.kbits <= 2)) and bk.bkv_fused_supported(lay, L, w.k)
    paths = [False] + ([True] if fused_ok else [])
    results = {}
    for one in paths:
        print(f"[case] {w.name} path {'fused' if one else 'separate'}", flush=True)
        gc = bk.allocate_cache(lay, shadow_on_host=(shadow == "host"))
        bk.kv_pack_append(lay, gc, P.to_dev(inp.K), P.to_dev(inp.V), L - 1, [0] * w.B)
        st = DecodeStep(lay, w.k, L, one_launch=one)
        out = st.step(gc, P.to_dev(inp.q), P.to_dev(kn[0]), P.to_dev(vn[0]), [L - 1] * w.B)
        torch.cuda.synchronize()
        assert st.ran_fused == one, "the fused step fell back to the separate launches"
        results[one] = dict(
            out=out.cpu().numpy().reshape(w.B, w.Hq, 128),
            sig=st.sigma.cpu().numpy().reshape(units, cap),
            idx=st.idx.cpu().numpy().reshape(units, w.k),
            buf={n: unit_slices(getattr(gc, n).cpu().numpy().view(np.uint8), units)
                 for n in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow")})
        del gc, st
    # the sampled units, stacked as the KV heads of one oracle batch row
    bh = [divmod(u, w.Hkv) for u in sample]
    n = len(sample)
    oracle.set_threads(min(n, 16))
    oc = oracle.Cache(oracle.Shape(1, w.G * n, n, 128, w.kbits, w.vbits, w.group, cap, w.key_format))
    oc.append(np.stack([inp.K[b, h] for b, h in bh])[None], np.stack([inp.V[b, h] for b, h in bh])[None],
              np.zeros(1, np.int32))
    oc.append(np.stack([kn[0][b, h] for b, h in bh])[None], np.stack([vn[0][b, h] for b, h in bh])[None],
              np.array([L - 1], np.int32))
    q = np.concatenate([inp.q[b, h * w.G:(h + 1) * w.G] for b, h in bh])[None]
    ref = oc.decode(q, np.array([L], np.int32), w.k, qbits=w.query_bits)
    ob = P.orc_buffers(oc)
    worst = {}
    def margin(tag, got, ref):
        e = np.abs(np.asarray(got, np.float64) - ref)
        tol = np.maximum(P.ATOL, P.RTOL * np.abs(ref))
        worst[tag] = max(worst.get(tag, 0.0), float((e / tol).max()))
    for one, r in results.items():
        tag = "fused" if one else "separate"
        for j, u in enumerate(sample):
            b, h = bh[j]
            for bname, arr in ob.items():
                per = arr.size // n
                assert np.array_equal(r["buf"][bname][u], arr[j * per:(j + 1) * per]), (tag, bname, u)
            np.testing.assert_allclose(r["sig"][u, :L], ref["sigma"][0, j, :L], rtol=1e-5, atol=2e-5)
            assert np.array_equal(r["idx"][u], oracle.topk(r["sig"][u, :L].astype(np.float64), w.k)), (tag, u)
            P.assert_topk_near_tie(r["idx"][u], ref["idx"][0, j], ref["sigma"][0, j], L, f"{tag} unit {u}")
            if w.planted and w.kbits >= 3:  # (1- and 2-bit keys may rank a planted token lower)
                assert set(inp.planted_pos[b, h].tolist()) <= set(r["idx"][u].tolist()), (tag, u)
            P.assert_close(r["out"][b, h * w.G:(h + 1) * w.G], ref["out"][0, j * w.G:(j + 1) * w.G],
                           f"{tag} unit {u} vs oracle(S_oracle)")
            margin(tag + " vs oracle(S_oracle)", r["out"][b, h * w.G:(h + 1) * w.G],
                   ref["out"][0, j * w.G:(j + 1) * w.G])
        # on the GPU's own selected sets
        sel = np.stack([r["idx"][u] for u in sample])[None]
        ref_s = oc.decode(q, np.array([L], np.int32), w.k, sel=sel, qbits=w.query_bits)
        for j, u in enumerate(sample):
            b, h = bh[j]
            P.assert_close(r["out"][b, h * w.G:(h + 1) * w.G], ref_s["out"][0, j * w.G:(j + 1) * w.G],
                           f"{tag} unit {u} vs oracle(S_gpu)")
            margin(tag + " vs oracle(S_gpu)", r["out"][b, h * w.G:(h + 1) * w.G],
                   ref_s["out"][0, j * w.G:(j + 1) * w.G])
    print(f"[margin] {w.name} ({shadow} shadow, {len(sample)} units): worst |error| / tolerance " +
          ", ".join(f"{k} {v:.3f}" for k, v in sorted(worst.items())), flush=True)
