"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case prints its name before touching the GPU.  Sizes span several
32-token tiles, several splits and a ragged tail, and every supported
(key bits, value bits, GQA group) combination.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

COMBOS = [(kb, vb, G) for kb in (4, 3) for vb in (4, 2) for G in (4, 8)]
# the low-bit codecs of the TailorKV review (1- and 2-bit keys) and groups of 64
CODECS = [(2, 2, 4, 64), (1, 2, 8, 64), (2, 4, 8, 32), (1, 4, 4, 32), (4, 4, 4, 64), (3, 2, 8, 64)]


@pytest.fixture(scope="module")
def P(orc):
    import parity
    return parity


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("kb,vb,g", [(4, 4, 32), (3, 2, 32), (4, 2, 32), (3, 4, 32), (2, 2, 32), (1, 4, 32),
                                     (2, 2, 64), (1, 2, 64), (4, 4, 64), (3, 2, 64)])
def test_pack_bit_exact(P, kb, vb, g):
    """Bulk prefill into a partial tile, a multi-token append with ragged
    positions (one sequence rewrites slots), then a single-token append."""
    import torch
    from bit_kv_attention_amd import binding as bk
    import oracle
    banner(f"pack kb={kb} vb={vb} g={g}")
    w = P.Workload("pack", 2, 8, 2, 128, 200, kb, vb, g, 8, 3, 31)
    inp = P.make_inputs(w, L=120)
    cap = 160
    lay = bk.make_layout(2, 8, 2, cap, kb, vb, group=g)
    gc = bk.allocate_cache(lay)
    oc = oracle.Cache(oracle.Shape(2, 8, 2, 128, kb, vb, g, cap))
    steps = [(inp.K[:, :, :77], inp.V[:, :, :77], [0, 0]),
             (inp.K[:, :, 77:117], inp.V[:, :, 77:117], [77, 60]),
             (inp.K[:, :, 117:118], inp.V[:, :, 117:118], [117, 100])]
    for Kn, Vn, pos in steps:
        bk.kv_pack_append(lay, gc, P.to_dev(Kn), P.to_dev(Vn), Kn.shape[2], pos)
        oc.append(Kn, Vn, np.array(pos, np.int32))
    torch.cuda.synchronize()
    g, o = P.gpu_buffers(gc), P.orc_buffers(oc)
    for name in g:
        assert np.array_equal(g[name], o[name]), name


def special_rows(rng, n):
    """fp16 rows [n, 128] whose groups hit the quantiser's edge cases:
    constant groups (step 0), a zero minimum met as -0 before +0 and as +0
    before -0 (the stored zero point keeps the first one's sign), the fp16
    extremes, a range so small that the fp16 step underflows to 0, and one
    value apart from an otherwise constant group."""
    x = rng.standard_normal((n, 128)).astype(np.float16)
    for t in range(n):
        case = t % 6
        g = (t // 6) % 4
        sl = slice(32 * g, 32 * g + 32)
        if case == 0:
            x[t, sl] = np.float16(1.5)
        elif case == 1:
            x[t, sl] = np.abs(x[t, sl]) + np.float16(0.5)
            x[t, 32 * g + 3] = np.float16(-0.0)
            x[t, 32 * g + 20] = np.float16(0.0)
        elif case == 2:
            x[t, sl] = np.abs(x[t, sl]) + np.float16(0.5)
            x[t, 32 * g + 9] = np.float16(0.0)
            x[t, 32 * g + 30] = np.float16(-0.0)
        elif case == 3:
            x[t, 32 * g] = np.float16(65504.0)
            x[t, 32 * g + 31] = np.float16(-65504.0)
        elif case == 4:
            x[t, sl] = np.float16(2.0 ** -14)
            x[t, 32 * g + 17] = np.float16(2.0 ** -14 + 2.0 ** -24)
        else:
            x[t, sl] = np.float16(-3.0)
            x[t, 32 * g + (t % 32)] = np.float16(7.25)
    return x


@pytest.mark.parametrize("kb,vb,g", [(4, 4, 32), (3, 2, 32), (2, 2, 64), (1, 2, 64)])
def test_pack_special_values(P, kb, vb, g):
    """Edge-value groups, bulk then one token at a time, bit-exact."""
    import torch
    from bit_kv_attention_amd import binding as bk
    import oracle
    banner(f"pack special values kb={kb} vb={vb} g={g}")
    rng = np.random.default_rng(7)
    B, Hkv, n, cap = 2, 2, 48, 64
    K = special_rows(rng, B * Hkv * n).reshape(B, Hkv, n, 128)
    V = special_rows(rng, B * Hkv * n)[::-1].copy().reshape(B, Hkv, n, 128)
    lay = bk.make_layout(B, 4 * Hkv, Hkv, cap, kb, vb, group=g)
    gc = bk.allocate_cache(lay)
    oc = oracle.Cache(oracle.Shape(B, 4 * Hkv, Hkv, 128, kb, vb, g, cap))
    steps = [(0, 40)] + [(t, t + 1) for t in range(40, n)]
    for a, e in steps:
        Kn, Vn = K[:, :, a:e], V[:, :, a:e]
        bk.kv_pack_append(lay, gc, P.to_dev(Kn), P.to_dev(Vn), e - a, [a, a])
        oc.append(Kn, Vn, np.array([a, a], np.int32))
    torch.cuda.synchronize()
    g, o = P.gpu_buffers(gc), P.orc_buffers(oc)
    for name in g:
        assert np.array_equal(g[name], o[name]), name


@pytest.mark.parametrize("kb,vb,G,g", [c + (32,) for c in COMBOS] + CODECS)
def test_step_parity_small(P, kb, vb, G, g):
    banner(f"step kb={kb} vb={vb} G={G} g={g}")
    w = P.Workload("small", 2, 2 * G, 2, 128, 1000, kb, vb, g, 24, 6, 100 + 10 * kb + vb + G + g)
    pair = P.build_pair(w, L=1000, cap=1024)
    lens = np.array([1000, 651])
    k = 24
    r = P.run_step(pair, lens, k)
    orc = pair["oc"].decode(pair["q"], lens, k, want_approx=True)
    for b in range(w.B):
        n = lens[b]
        np.testing.assert_allclose(r["sigma"][b, :, :n], orc["sigma"][b, :, :n], rtol=1e-5, atol=2e-5)
        assert np.all(np.isneginf(r["sigma"][b, :, n:((n + 31) // 32) * 32]))
    # top-k: exact against the oracle's selection on the GPU's own scores ...
    import oracle
    for b in range(w.B):
        for h in range(w.Hkv):
            n = lens[b]
            want = oracle.topk(r["sigma"][b, h, :n].astype(np.float64), k)
            assert np.array_equal(r["idx"][b, h], want), (b, h)
            P.assert_topk_near_tie(r["idx"][b, h], orc["idx"][b, h], orc["sigma"][b, h], n, f"b{b}h{h}")
    # ... outputs against the oracle on the GPU's set and on its own set
    orc_s = pair["oc"].decode(pair["q"], lens, k, sel=r["idx"])
    P.assert_close(r["out"], orc_s["out"], "out vs oracle(S_gpu)")
    P.assert_close(r["out"], orc["out"], "out vs oracle(S_oracle)")


@pytest.mark.parametrize("kb,vb,G", [(4, 4, 4), (3, 2, 8)])
def test_approx_only_and_exact(P, kb, vb, G):
    """k = 0 is the approximate output; k = len and k > len the exact one."""
    banner(f"k=0/k=L kb={kb} vb={vb} G={G}")
    w = P.Workload("ends", 2, 2 * G, 2, 128, 700, kb, vb, 32, 0, 4, 7 + G)
    pair = P.build_pair(w, L=700, cap=704)
    lens = np.array([700, 333])
    r0 = P.run_step(pair, lens, 0)
    orc = pair["oc"].decode(pair["q"], lens, 0, want_approx=True, want_exact=True)
    P.assert_close(r0["out"], orc["out_approx"], "k=0")
    from bit_kv_attention_amd.step import DecodeStep
    import torch
    for k in (700, 5000):
        st = DecodeStep(pair["lay"], k, 700)
        out = st.attend(pair["gc"], P.to_dev(pair["q"]), lens)
        torch.cuda.synchronize()
        P.assert_close(out.cpu().numpy().reshape(w.B, w.Hq, 128), orc["out_exact"], f"k={k}")
        idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, k)
        for b in range(w.B):
            assert idx[b, :, :lens[b]].tolist() == [list(range(lens[b]))] * w.Hkv
            assert np.all(idx[b, :, lens[b]:] == -1)


def test_edge_lengths(P):
    """len 0, 1, 31, 33 and one long ragged sequence in one batch."""
    banner("edge lengths")
    w = P.Workload("edge", 5, 8, 2, 128, 1100, 3, 2, 32, 16, 2, 55)
    pair = P.build_pair(w, L=1100, cap=1120)
    lens = np.array([0, 1, 31, 33, 1100])
    r = P.run_step(pair, lens, 16)
    orc = pair["oc"].decode(pair["q"], lens, 16)
    assert np.all(r["out"][0] == 0)
    assert np.all(r["idx"][0] == -1)
    for b in range(1, 5):
        for h in range(w.Hkv):
            P.assert_topk_near_tie(r["idx"][b, h], orc["idx"][b, h], orc["sigma"][b, h], lens[b], f"b{b}")
    orc_s = pair["oc"].decode(pair["q"], lens, 16, sel=np.where(r["idx"] < 0, -1, r["idx"]))
    P.assert_close(r["out"], orc_s["out"], "out vs oracle(S_gpu)")


def test_ties_take_lower_index(P):
    """Identical key rows give identical scores: the selected set must be the
    lowest indices among the tied tokens."""
    banner("ties")
    import torch
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    rng = np.random.default_rng(3)
    L, cap = 300, 320
    row = rng.standard_normal(128).astype(np.float16)
    K = np.tile(row, (1, 1, L, 1))
    K[0, 0, 250] = (row.astype(np.float32) * 2).astype(np.float16)  # one clear winner
    V = rng.standard_normal((1, 1, L, 128)).astype(np.float16)
    q = rng.standard_normal((1, 4, 128)).astype(np.float16)
    lay = bk.make_layout(1, 4, 1, cap, 4, 4)
    gc = bk.allocate_cache(lay)
    bk.kv_pack_append(lay, gc, P.to_dev(K), P.to_dev(V), L, [0])
    st = DecodeStep(lay, 10, L)
    st.attend(gc, P.to_dev(q), [L])
    torch.cuda.synchronize()
    idx = st.idx.cpu().numpy()[:10].tolist()
    sig = st.sigma.cpu().numpy()[:L]
    others = [t for t in range(L) if t != 250]
    assert np.all(sig[others] == sig[0])
    want = sorted([250] + others[:9]) if sig[250] > sig[0] else others[:10]
    assert idx == want


@pytest.mark.parametrize("L,k", [(10000, 50), (5000, 4999), (4100, 1)])
def test_topk_bucket_overflow_fallback(P, L, k):
    """All keys equal: every score lands in the threshold bucket, more
    candidates than the in-LDS list holds, so the selection falls back to
    re-reading the scores; ties must resolve to the lowest indices."""
    banner(f"top-k overflow L={L} k={k}")
    import torch
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    rng = np.random.default_rng(5)
    cap = ((L + 31) // 32) * 32
    row = rng.standard_normal(128).astype(np.float16)
    K = np.tile(row, (1, 1, L, 1))
    V = rng.standard_normal((1, 1, L, 128)).astype(np.float16)
    q = rng.standard_normal((1, 8, 128)).astype(np.float16)
    lay = bk.make_layout(1, 8, 1, cap, 3, 2)
    gc = bk.allocate_cache(lay)
    bk.kv_pack_append(lay, gc, P.to_dev(K), P.to_dev(V), L, [0])
    st = DecodeStep(lay, k, L)
    out = st.attend(gc, P.to_dev(q), [L])
    torch.cuda.synchronize()
    sig = st.sigma.cpu().numpy()[:L]
    assert np.all(sig == sig[0])
    assert st.idx.cpu().numpy()[:k].tolist() == list(range(k))
    # equal keys: the output is the weighted mean with exact values for the
    # first k tokens and dequantised ones for the rest
    import oracle
    oc = oracle.Cache(oracle.Shape(1, 8, 1, 128, 3, 2, 32, cap))
    oc.append(K, V, np.zeros(1, np.int32))
    ref = oc.decode(q, np.array([L], np.int32), k, sel=st.idx.cpu().numpy()[:k].reshape(1, 1, k))
    P.assert_close(out.cpu().numpy().reshape(1, 8, 128), ref["out"], "equal keys")


def test_many_correction_chunks(P):
    """k >= len at 17000 tokens: 532 correction chunks per head (more than one
    LDS batch in the merge), the output is exact attention."""
    banner("k=L at 17000 tokens")
    w = P.Workload("bigk", 1, 4, 1, 128, 17000, 3, 2, 32, 17000, 4, 21)
    pair = P.build_pair(w, L=17000, cap=17024)
    lens = np.array([17000])
    r = P.run_step(pair, lens, 17000)
    orc = pair["oc"].decode(pair["q"], lens, 0, want_exact=True)
    P.assert_close(r["out"], orc["out_exact"], "k=L")
    assert r["idx"][0, 0].tolist() == list(range(17000))


@pytest.mark.parametrize("kb,vb,G", [(4, 4, 4), (3, 2, 8)])
def test_step_parity_multi_slice(P, kb, vb, G):
    """Few units and a long context: several top-k slices and scan splits per
    unit, so the cross-workgroup paths (histogram, candidates, bitmap) run."""
    banner(f"multi-slice kb={kb} vb={vb} G={G}")
    w = P.Workload("ms", 1, 2 * G, 2, 128, 6000, kb, vb, 32, 40, 8, 300 + G)
    pair = P.build_pair(w, L=6000, cap=6016)
    lens = np.array([6000])
    r = P.run_step(pair, lens, 40)
    orc = pair["oc"].decode(pair["q"], lens, 40)
    import oracle
    for h in range(w.Hkv):
        want = oracle.topk(r["sigma"][0, h, :6000].astype(np.float64), 40)
        assert np.array_equal(r["idx"][0, h], want)
        P.assert_topk_near_tie(r["idx"][0, h], orc["idx"][0, h], orc["sigma"][0, h], 6000, f"h{h}")
    orc_s = pair["oc"].decode(pair["q"], lens, 40, sel=r["idx"])
    P.assert_close(r["out"], orc_s["out"], "out vs oracle(S_gpu)")
    P.assert_close(r["out"], orc["out"], "out vs oracle(S_oracle)")


@pytest.mark.parametrize("L,k", [(32768, 256), (20000, 3000), (40000, 4000), (9000, 1)])
def test_topk_paths_on_given_scores(P, L, k):
    """topk_select on given scores with many exact ties, ragged lengths and two
    calls in a row on one workspace: the fused slice+merge launch (few
    candidate slots), the separate merge launch (many) and the
    single-workgroup kernel (too many for the merge), against the oracle's
    full sort."""
    banner(f"top-k paths L={L} k={k}")
    import torch
    import oracle
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    B, Hkv = 2, 2
    cap = ((L + 31) // 32) * 32
    lay = bk.make_layout(B, 4 * Hkv, Hkv, cap, 4, 4)
    rng = np.random.default_rng(L + k)
    sig = (np.round(rng.standard_normal((B, Hkv, cap)) * 64) / 64).astype(np.float32)  # many ties
    sig[:, :, ::97] = 3.5  # a tied block above the rest
    lens = [L, L // 3 + 5]
    st = DecodeStep(lay, k, L)
    st.sigma.copy_(torch.from_numpy(sig.reshape(-1)))
    for rep in range(2):
        st.idx.fill_(-7)
        bk.topk_select(lay, st.sigma, lens, k, st.idx, st.ws)
        torch.cuda.synchronize()
        idx = st.idx.cpu().numpy().reshape(B, Hkv, k)
        for b in range(B):
            for h in range(Hkv):
                want = oracle.topk(sig[b, h, :lens[b]].astype(np.float64), k)
                assert np.array_equal(idx[b, h], want), (rep, b, h)


@pytest.mark.parametrize("L,k,W", [(32768, 256, 64), (20000, 3000, 128), (40000, 4000, 32), (9000, 1, 16),
                                   (5000, 0, 100), (3000, 64, 5000), (6000, 40, 0)])
def test_topk_window_on_given_scores(P, L, k, W):
    """topk_select_window on given scores (many exact ties): the newest
    min(W, len) tokens always, the top-k over the rest, ascending, -1 fill --
    every top-k path, k = 0, a window longer than the sequence, len 0, and
    W = 0 equal to topk_select; two calls in a row on one workspace."""
    banner(f"top-k window L={L} k={k} W={W}")
    import torch
    import oracle
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    B, Hkv = 4, 2
    cap = ((L + 31) // 32) * 32
    lay = bk.make_layout(B, 4 * Hkv, Hkv, cap, 4, 4)
    rng = np.random.default_rng(L + k + W)
    sig = (np.round(rng.standard_normal((B, Hkv, cap)) * 64) / 64).astype(np.float32)
    sig[:, :, ::97] = 3.5
    lens = [L, L // 3 + 5, W // 2, 0]
    row = k + W
    st = DecodeStep(lay, k, L, window=W)
    st.sigma.copy_(torch.from_numpy(sig.reshape(-1)))
    for rep in range(2):
        st.idx.fill_(-7)
        bk.topk_select_window(lay, st.sigma, lens, k, W, st.idx, st.ws)
        torch.cuda.synchronize()
        idx = st.idx.cpu().numpy().reshape(B, Hkv, max(row, 1))[:, :, :row]
        for b in range(B):
            for h in range(Hkv):
                want = oracle.topk_window(sig[b, h, :lens[b]].astype(np.float64), k, W)
                assert np.array_equal(idx[b, h], want), (rep, b, h)
    if W == 0:
        st.idx.fill_(-7)
        bk.topk_select(lay, st.sigma, lens, k, st.idx, st.ws)
        torch.cuda.synchronize()
        assert np.array_equal(st.idx.cpu().numpy().reshape(B, Hkv, k), idx)


@pytest.mark.parametrize("kb,vb,G,W,fmt", [(4, 4, 4, 64, ""), (3, 2, 8, 200, ""), (4, 4, 4, 64, "q8"),
                                            (4, 2, 8, 100, "mx")])
def test_step_parity_window(P, kb, vb, G, W, fmt):
    """A whole step with a recent window: the GPU's rows against the oracle's
    selection on the GPU's scores (exact), the output against the oracle on
    the GPU's rows and on its own."""
    banner(f"step window kb={kb} vb={vb} G={G} W={W} {fmt}")
    qb, kf = (8 if fmt == "q8" else 0), {"mx": 2, "mx1": 1}.get(fmt, 0)
    import torch
    import oracle
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("win", 3, 2 * G, 2, 128, 3000, kb, vb, 32, 32, 6, 500 + G + W, query_bits=qb, key_format=kf)
    pair = P.build_pair(w, L=3000, cap=3008)
    lens = np.array([3000, 1234, W // 3])
    k = 32
    pos = [int(x) - 1 for x in lens]
    from bit_kv_attention_amd import binding as bk
    bk.kv_pack_append(pair["lay"], pair["gc"], P.to_dev(pair["k1"]), P.to_dev(pair["v1"]), 1, pos)
    pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
    st = DecodeStep(pair["lay"], k, 3000, window=W)
    out = st.attend(pair["gc"], P.to_dev(pair["q"]), lens)
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(w.B, w.Hq, 128)
    sigma = st.sigma.cpu().numpy().reshape(w.B, w.Hkv, pair["cap"])
    idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, k + W)
    orc = pair["oc"].decode(pair["q"], lens, 0, want_approx=True, qbits=qb)
    sel_o = np.full_like(idx, -1)
    for b in range(w.B):
        n = lens[b]
        np.testing.assert_allclose(sigma[b, :, :n], orc["sigma"][b, :, :n], rtol=1e-5, atol=2e-5)
        for h in range(w.Hkv):
            want = oracle.topk_window(sigma[b, h, :n].astype(np.float64), k, W)
            assert np.array_equal(idx[b, h], want), (b, h)
            sel_o[b, h] = oracle.topk_window(orc["sigma"][b, h, :n], k, W)
            kk = min(k, n - min(W, n))  # the selected part of the row
            P.assert_topk_near_tie(idx[b, h, :kk], sel_o[b, h, :kk], orc["sigma"][b, h], n - min(W, n), f"b{b}h{h}")
    orc_s = pair["oc"].decode(pair["q"], lens, k + W, sel=idx, qbits=qb)
    P.assert_close(out, orc_s["out"], "out vs oracle(rows_gpu)")
    orc_o = pair["oc"].decode(pair["q"], lens, k + W, sel=sel_o, qbits=qb)
    P.assert_close(out, orc_o["out"], "out vs oracle(rows_oracle)")


@pytest.mark.parametrize("L,nb,bs,ties", [(32768, 16, 128, False), (32768, 16, 128, True), (131072, 64, 128, True),
                                          (40000, 3, 1024, False), (9000, 70, 32, True), (5000, 50, 128, False),
                                          (6000, 7, 512, True)])
def test_topk_blocks_on_given_scores(P, L, nb, bs, ties):
    """topk_select_blocks on given scores against the oracle: distinct and
    massively tied block scores (the select's fallback), a budget covering
    every block, blocks longer than one load, a ragged last block, len 0;
    two calls in a row."""
    banner(f"block top-k L={L} nb={nb} bs={bs} ties={ties}")
    import torch
    import oracle
    from bit_kv_attention_amd import binding as bk
    B, Hkv = 3, 2
    cap = ((L + 31) // 32) * 32
    lay = bk.make_layout(B, 4 * Hkv, Hkv, cap, 4, 4)
    rng = np.random.default_rng(L + nb + bs)
    if ties:
        sig = (np.round(rng.standard_normal((B, Hkv, cap)) * 64) / 64).astype(np.float32)
        sig[:, :, ::97] = 3.5  # nearly every block ties at the top
    else:
        sig = rng.standard_normal((B, Hkv, cap)).astype(np.float32)
    lens = [L, L // 3 + 5, 0]
    row = nb * bs
    sigd = torch.from_numpy(sig.reshape(-1)).cuda()
    idxd = torch.empty(B * Hkv * row, dtype=torch.int32, device="cuda")
    ws = torch.zeros((bk.bkv_workspace_bytes(lay, L, row) + 3) // 4, dtype=torch.float32, device="cuda")
    for rep in range(2):
        idxd.fill_(-7)
        bk.topk_select_blocks(lay, sigd, lens, nb, bs, idxd, ws)
        torch.cuda.synchronize()
        idx = idxd.cpu().numpy().reshape(B, Hkv, row)
        for b in range(B):
            for h in range(Hkv):
                want = oracle.topk_blocks(sig[b, h, :lens[b]].astype(np.float64), nb, bs)
                assert np.array_equal(idx[b, h], want), (rep, b, h)


@pytest.mark.parametrize("kb,vb,G,nb,bs,fmt", [(4, 4, 4, 6, 128, ""), (3, 2, 8, 20, 32, ""),
                                               (2, 2, 8, 10, 64, "q8"), (4, 4, 4, 6, 128, "mx")])
def test_step_parity_blocks(P, kb, vb, G, nb, bs, fmt):
    """A whole step with block selection: the GPU's rows against the oracle's
    block selection on the GPU's scores (exact) and on its own (chosen blocks
    may differ only by near-ties of the block score), the output against the
    oracle on both rows."""
    banner(f"step blocks kb={kb} vb={vb} G={G} nb={nb} bs={bs} {fmt}")
    qb, kf = (8 if fmt == "q8" else 0), {"mx": 2, "mx1": 1}.get(fmt, 0)
    import torch
    import oracle
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("blk", 3, 2 * G, 2, 128, 3000, kb, vb, 32, 32, 6, 700 + G + nb, query_bits=qb, key_format=kf)
    pair = P.build_pair(w, L=3000, cap=3008)
    lens = np.array([3000, 1234, 77])
    pos = [int(x) - 1 for x in lens]
    bk.kv_pack_append(pair["lay"], pair["gc"], P.to_dev(pair["k1"]), P.to_dev(pair["v1"]), 1, pos)
    pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
    st = DecodeStep(pair["lay"], nb, 3000, block=bs)
    out = st.attend(pair["gc"], P.to_dev(pair["q"]), lens)
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(w.B, w.Hq, 128)
    sigma = st.sigma.cpu().numpy().reshape(w.B, w.Hkv, pair["cap"])
    idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, nb * bs)
    orc = pair["oc"].decode(pair["q"], lens, 0, want_approx=True, qbits=qb)
    sel_o = np.full_like(idx, -1)
    for b in range(w.B):
        n = lens[b]
        np.testing.assert_allclose(sigma[b, :, :n], orc["sigma"][b, :, :n], rtol=1e-5, atol=2e-5)
        nblk = -(-n // bs)
        for h in range(w.Hkv):
            want = oracle.topk_blocks(sigma[b, h, :n].astype(np.float64), nb, bs)
            assert np.array_equal(idx[b, h], want), (b, h)
            sel_o[b, h] = oracle.topk_blocks(orc["sigma"][b, h, :n], nb, bs)
            bscore = np.array([orc["sigma"][b, h, j * bs:min(n, j * bs + bs)].max() for j in range(nblk)])
            kbk = min(nb, nblk)
            P.assert_topk_near_tie(idx[b, h, ::bs][:kbk] // bs, sel_o[b, h, ::bs][:kbk] // bs, bscore, nblk,
                                   f"b{b}h{h}")
    orc_s = pair["oc"].decode(pair["q"], lens, nb * bs, sel=idx, qbits=qb)
    P.assert_close(out, orc_s["out"], "out vs oracle(rows_gpu)")
    orc_o = pair["oc"].decode(pair["q"], lens, nb * bs, sel=sel_o, qbits=qb)
    P.assert_close(out, orc_o["out"], "out vs oracle(rows_oracle)")


@pytest.mark.parametrize("kb,vb,G,nb,bs", [(4, 4, 4, 24, 128), (3, 2, 8, 40, 64)])
def test_step_parity_blocks_long_rows(P, kb, vb, G, nb, bs):
    """Block rows long enough that each correction workgroup walks several
    consecutive chunks (32 units, thousands of selected tokens per unit), with
    ragged lengths: a short sequence whose row ends in -1 entries mid-record,
    and one shorter than a single block.  Output against the oracle on the
    GPU's rows."""
    banner(f"step blocks long rows kb={kb} vb={vb} G={G} nb={nb} bs={bs}")
    import torch
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("blkl", 4, 8 * G, 8, 128, 6000, kb, vb, 32, 32, 6, 900 + G + nb)
    pair = P.build_pair(w, L=6000, cap=6016)
    lens = np.array([6000, 4321, 1000, 50])
    pos = [int(x) - 1 for x in lens]
    bk.kv_pack_append(pair["lay"], pair["gc"], P.to_dev(pair["k1"]), P.to_dev(pair["v1"]), 1, pos)
    pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
    st = DecodeStep(pair["lay"], nb, 6000, block=bs)
    out = st.attend(pair["gc"], P.to_dev(pair["q"]), lens)
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(w.B, w.Hq, 128)
    idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, nb * bs)
    assert (nb * bs // 32) * w.B * w.Hkv > 1024  # several chunks per correction workgroup
    orc_s = pair["oc"].decode(pair["q"], lens, nb * bs, sel=idx)
    P.assert_close(out, orc_s["out"], "out vs oracle(rows_gpu)")
    # and the plain top-k with the same long rows (k well past 32 chunks)
    st2 = DecodeStep(pair["lay"], nb * bs, 6000)
    out2 = st2.attend(pair["gc"], P.to_dev(pair["q"]), lens)
    torch.cuda.synchronize()
    idx2 = st2.idx.cpu().numpy().reshape(w.B, w.Hkv, nb * bs)
    orc2 = pair["oc"].decode(pair["q"], lens, nb * bs, sel=idx2)
    P.assert_close(out2.cpu().numpy().reshape(w.B, w.Hq, 128), orc2["out"], "top-k long rows vs oracle(S_gpu)")


@pytest.mark.parametrize("kb,vb,G,g,fmt", [c + (32, "") for c in COMBOS] + [(2, 2, 4, 64, ""), (1, 2, 8, 64, ""),
                                            (4, 4, 4, 32, "q8"), (2, 2, 8, 64, "q8"),
                                            (4, 2, 4, 32, "mx"), (4, 4, 8, 32, "mx1")])
def test_decode_select_equals_two_calls(P, kb, vb, G, g, fmt):
    """qattn_decode_select (selection inside the scan's launch) against
    qattn_decode_approx + topk_select on the same inputs: identical sigma, rows
    and output, rows exact against the oracle's top-k of that sigma; ragged and
    empty sequences, k = 1, k >= len, and a budget past the in-launch limit
    (two launches)."""
    banner(f"decode_select kb={kb} vb={vb} G={G} g={g} {fmt}")
    qb, kf = (8 if fmt == "q8" else 0), {"mx": 2, "mx1": 1}.get(fmt, 0)
    import torch
    import oracle
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("sel", 4, 2 * G, 2, 128, 4000, kb, vb, g, 32, 6, 900 + 10 * kb + vb + G, query_bits=qb,
                   key_format=kf)
    pair = P.build_pair(w, L=4000, cap=4000)
    lens = np.array([3999, 2500, 1, 0])  # (the prefill filled 3999 slots)
    q = P.to_dev(pair["q"])
    for k in (1, 37, 300, 500, 2600, 5000):  # 16 ranges per unit: 500 is the last in-launch budget
        runs = []
        for fused in (True, False):  # the selection in the scan's launch whenever possible, and two calls
            st = DecodeStep(pair["lay"], k, 3999, fused=fused, select_mode=1, exclude=False, one_launch=False)
            for _ in range(2):  # twice on one workspace
                st.sigma.fill_(float("nan"))
                st.idx.fill_(-7)
                out = st.attend(pair["gc"], q, lens)
            torch.cuda.synchronize()
            runs.append((st.sigma.cpu().numpy().reshape(w.B, w.Hkv, -1), st.idx.cpu().numpy().reshape(w.B, w.Hkv, k),
                         out.cpu().numpy()))
        (s1, i1, o1), (s0, i0, o0) = runs
        for b in range(w.B):
            n = lens[b]
            assert np.array_equal(s1[b, :, :n], s0[b, :, :n]), (k, b)
            for h in range(w.Hkv):
                want = oracle.topk(s1[b, h, :n].astype(np.float64), k)
                assert np.array_equal(i1[b, h], want), (k, b, h)
        assert np.array_equal(i1, i0), k
        assert np.array_equal(o1, o0), k
        if fmt and k == 37:  # the in-launch scores are the codec's own
            orc = pair["oc"].decode(pair["q"], lens, k, qbits=qb)
            for b in range(w.B):
                n = lens[b]
                np.testing.assert_allclose(s1[b, :, :n], orc["sigma"][b, :, :n], rtol=1e-5, atol=2e-5)


@pytest.mark.parametrize("kb,vb,G,fmt", [(4, 4, 4, ""), (3, 2, 8, ""), (3, 4, 4, "q8"), (4, 2, 8, "mx")])
def test_hybrid_host_correction(P, kb, vb, G, fmt):
    """The exact half of the correction on the host (qattn_exact_host over a
    pinned host shadow) merged on the GPU (qattn_correct_hybrid): output
    against the oracle on the GPU's rows, and against the all-GPU correction;
    ragged and empty sequences, k >= len, k = 0."""
    banner(f"hybrid host correction kb={kb} vb={vb} G={G} {fmt}")
    qb, kf = (8 if fmt == "q8" else 0), {"mx": 2, "mx1": 1}.get(fmt, 0)
    import torch
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("hyb", 3, 2 * G, 2, 128, 2000, kb, vb, 32, 48, 6, 1200 + G)
    inp = P.make_inputs(w, L=1999)
    lay = bk.make_layout(w.B, w.Hq, w.Hkv, 2016, kb, vb, query_bits=qb, key_format=kf)
    hc = bk.allocate_cache(lay, shadow_on_host=True)
    bk.kv_pack_append(lay, hc, P.to_dev(inp.K), P.to_dev(inp.V), 1999, [0] * w.B)
    import oracle
    oc = oracle.Cache(oracle.Shape(w.B, w.Hq, w.Hkv, 128, kb, vb, 32, 2016, kf))
    oc.append(inp.K, inp.V, np.zeros(w.B, np.int32))
    lens = np.array([1999, 777, 0])
    q = P.to_dev(inp.q)
    for k in (48, 1000, 0):
        st = DecodeStep(lay, k, 1999, one_launch=False)
        out_h = st.attend_hybrid(hc, q, lens, n_threads=4).clone()
        torch.cuda.synchronize()
        idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, max(k, 1))[:, :, :k]
        out_g = st.attend(hc, q, lens)
        torch.cuda.synchronize()
        oh = out_h.cpu().numpy().reshape(w.B, w.Hq, 128)
        og = out_g.cpu().numpy().reshape(w.B, w.Hq, 128)
        orc = oc.decode(inp.q, lens, k, sel=idx if k > 0 else None, qbits=qb)
        P.assert_close(oh, orc["out"], f"hybrid vs oracle k={k}")
        np.testing.assert_allclose(oh, og, rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("kb,vb,G", [(4, 4, 4), (3, 2, 8)])
def test_hybrid_pipeline_layers(P, kb, vb, G):
    """HybridPipeline: three layers of the hybrid step over two micro-batches,
    each micro-batch's host pass overlapping the other's GPU work: every
    layer's output against the all-GPU step on a copy of that layer's cache
    and against the oracle end to end (the appended token included, ragged
    lengths)."""
    banner(f"hybrid pipeline kb={kb} vb={vb} G={G}")
    import torch
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep, HybridPipeline
    import oracle
    nl, L, cap, k = 3, 1500, 1504, 40
    pos = [1499, 1100, 640, 3]
    lens = np.array(pos) + 1
    caches, refs, orcs, qs, kns, vns, outs, ins = [], [], [], [], [], [], [], []
    for i in range(nl):
        w = P.Workload("hypipe", 4, 2 * G, 2, 128, L, kb, vb, 32, k, 4, 1300 + 10 * i + G)
        inp = P.make_inputs(w, L=L - 1)
        kn, vn = P.make_new_tokens(w, 1, inp.outlier_ch)
        lay = bk.make_layout(w.B, w.Hq, w.Hkv, cap, kb, vb)
        hc = bk.allocate_cache(lay, shadow_on_host=True)
        bk.kv_pack_append(lay, hc, P.to_dev(inp.K), P.to_dev(inp.V), L - 1, [0] * w.B)
        gc = bk.allocate_cache(lay)
        for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow"):
            getattr(gc, name).copy_(getattr(hc, name))
        oc = oracle.Cache(oracle.Shape(w.B, w.Hq, w.Hkv, 128, kb, vb, 32, cap))
        oc.append(inp.K, inp.V, np.zeros(w.B, np.int32))
        oc.append(kn[0], vn[0], np.array(pos, np.int32))
        caches.append(hc), refs.append(gc), orcs.append(oc), ins.append(inp)
        qs.append(P.to_dev(inp.q)), kns.append(P.to_dev(kn[0])), vns.append(P.to_dev(vn[0]))
        outs.append(torch.full((w.B * w.Hq * 128,), float("nan"), dtype=torch.float32, device="cuda"))
    pipe = HybridPipeline(lay, k, L, micro=2, n_threads=4)
    pipe.run(caches, qs, kns, vns, pos, outs)
    torch.cuda.synchronize()
    for i in range(nl):
        st = DecodeStep(lay, k, L, one_launch=False)
        og = st.step(refs[i], qs[i], kns[i], vns[i], pos)
        torch.cuda.synchronize()
        oh = outs[i].cpu().numpy().reshape(4, 2 * G, 128)
        np.testing.assert_allclose(oh, og.cpu().numpy().reshape(4, 2 * G, 128), rtol=1e-4, atol=1e-5)
        # the appended token reached the host shadow of both micro-batches
        for name in ("k_shadow", "v_shadow"):
            assert torch.equal(getattr(caches[i], name), getattr(refs[i], name).cpu()), (i, name)
        orc = orcs[i].decode(ins[i].q, lens, k)
        P.assert_close(oh, orc["out"], f"layer {i} vs oracle(S_oracle)")


@pytest.mark.parametrize("kb,vb,G,g", [(4, 4, 4, 32), (3, 2, 8, 32), (2, 2, 8, 64), (1, 2, 4, 64), (1, 4, 8, 32)])
def test_exclude_path(P, kb, vb, G, g):
    """qattn_decode_unselected + qattn_correct_unselected (the unselected
    tokens' approximate state merged with the selected tokens' exact terms)
    against the oracle on the GPU's rows; ragged and empty sequences, k >= len,
    k = 0, two calls in a row; for 3- and 4-bit keys also against the
    subtracting qattn_correct."""
    banner(f"exclude path kb={kb} vb={vb} G={G} g={g}")
    import torch
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("exc", 3, 2 * G, 2, 128, 3000, kb, vb, g, 40, 6, 1300 + 10 * kb + G + g)
    pair = P.build_pair(w, L=3000, cap=3008)
    lens = np.array([2999, 1400, 0])
    q = P.to_dev(pair["q"])
    for k in (40, 1500, 0):
        st = DecodeStep(pair["lay"], k, 2999, exclude=True)
        for _ in range(2):
            out = st.attend(pair["gc"], q, lens)
        torch.cuda.synchronize()
        o = out.cpu().numpy().reshape(w.B, w.Hq, 128)
        idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, max(k, 1))[:, :, :k]
        orc = pair["oc"].decode(pair["q"], lens, k, sel=idx if k > 0 else None)
        P.assert_close(o, orc["out"], f"exclude vs oracle k={k}")
        if kb >= 3:
            st2 = DecodeStep(pair["lay"], k, 2999, exclude=False)
            o2 = st2.attend(pair["gc"], q, lens)
            torch.cuda.synchronize()
            np.testing.assert_allclose(o, o2.cpu().numpy().reshape(w.B, w.Hq, 128), rtol=2e-3, atol=2e-4)


@pytest.mark.parametrize("kb,vb,G,g", [(4, 4, 4, 32), (1, 2, 8, 64)])
def test_score_select_equals_decode_select(P, kb, vb, G, g):
    """qattn_score_select writes the same sigma and rows as qattn_decode_select,
    in the scan's launch and as two launches."""
    banner(f"score_select kb={kb} vb={vb} G={G} g={g}")
    import torch
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("ss", 3, 2 * G, 2, 128, 3000, kb, vb, g, 40, 6, 1500 + G + g)
    pair = P.build_pair(w, L=3000, cap=3008)
    lens = np.array([2999, 1400, 0])
    q = P.to_dev(pair["q"])
    for k in (40, 500):
        for mode in (1, 2):
            a = DecodeStep(pair["lay"], k, 2999)
            b = DecodeStep(pair["lay"], k, 2999)
            bk.qattn_decode_select(pair["lay"], pair["gc"], q, lens, k, a.sigma, a.idx, a.ws, mode=mode)
            bk.qattn_score_select(pair["lay"], pair["gc"], q, lens, k, b.sigma, b.idx, b.ws, mode=mode)
            torch.cuda.synchronize()
            sa = a.sigma.cpu().numpy().reshape(w.B, w.Hkv, -1)
            sb = b.sigma.cpu().numpy().reshape(w.B, w.Hkv, -1)
            for bb in range(w.B):
                assert np.array_equal(sa[bb, :, :lens[bb]], sb[bb, :, :lens[bb]]), (k, mode)
            assert torch.equal(a.idx, b.idx), (k, mode)


@pytest.mark.parametrize("kb,vb,G,g", [(4, 4, 4, 32), (3, 2, 8, 32), (4, 2, 8, 64), (2, 2, 4, 64), (1, 4, 8, 32)])
def test_decode_step_equals_append_then_select(P, kb, vb, G, g):
    """qattn_decode_step (the append inside the scan's launch) against
    kv_pack_append + qattn_decode_select on two copies of one cache: the
    cache bytes after the step are equal, and so are sigma, the rows and the
    corrected output; the new tokens sit at a split start, a tile start, the
    middle of a tile and slot 0; both selection modes; three steps in a row."""
    banner(f"decode_step kb={kb} vb={vb} G={G} g={g}")
    import torch
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("dstep", 4, 2 * G, 2, 128, 3000, kb, vb, g, 32, 6, 1700 + 10 * kb + G + g)
    inp = P.make_inputs(w, L=2900)
    lay = bk.make_layout(w.B, w.Hq, w.Hkv, 3008, kb, vb, group=g)
    caches = [bk.allocate_cache(lay) for _ in range(2)]
    pre = [2048, 1535, 1000, 0]  # tokens already in the cache per sequence
    for c in caches:
        bk.kv_pack_append(lay, c, P.to_dev(inp.K), P.to_dev(inp.V), 2900, [0] * w.B)
    knew, vnew = P.make_new_tokens(w, 3, inp.outlier_ch)
    q = P.to_dev(inp.q)
    for mode in (1, 2):
        steps = [DecodeStep(lay, w.k, 3008, select_mode=mode) for _ in range(2)]
        for i in range(3):
            lens = [p + 1 + i for p in pre]
            kn, vn = P.to_dev(knew[i]), P.to_dev(vnew[i])
            bk.qattn_decode_step(lay, caches[0], kn, vn, q, lens, w.k, steps[0].sigma, steps[0].idx, steps[0].ws,
                                 mode=mode)
            bk.kv_pack_append(lay, caches[1], kn, vn, 1, [n - 1 for n in lens])
            bk.qattn_decode_select(lay, caches[1], q, lens, w.k, steps[1].sigma, steps[1].idx, steps[1].ws, mode=mode)
            for st, c in zip(steps, caches):
                bk.qattn_correct(lay, c, q, lens, st.idx, w.k, st.ws, st.out)
            torch.cuda.synchronize()
            ga, gb = P.gpu_buffers(caches[0]), P.gpu_buffers(caches[1])
            for name in ga:
                assert np.array_equal(ga[name], gb[name]), (mode, i, name)
            sa = steps[0].sigma.cpu().numpy().reshape(w.B, w.Hkv, -1)
            sb = steps[1].sigma.cpu().numpy().reshape(w.B, w.Hkv, -1)
            for b in range(w.B):
                assert np.array_equal(sa[b, :, :lens[b]], sb[b, :, :lens[b]]), (mode, i, b)
            assert torch.equal(steps[0].idx, steps[1].idx), (mode, i)
            assert torch.equal(steps[0].out, steps[1].out), (mode, i)


@pytest.mark.parametrize("kb,vb,G,g,window,block", [(2, 2, 4, 64, 50, 0), (1, 2, 8, 64, 0, 64), (4, 4, 4, 32, 0, 128)])
def test_exclude_path_window_and_blocks(P, kb, vb, G, g, window, block):
    """The exclusion path with a recent window and with block selection: the
    output against the oracle on the GPU's rows (k + window, or n_blocks *
    block entries)."""
    banner(f"exclude path kb={kb} vb={vb} G={G} g={g} window={window} block={block}")
    import torch
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("excwb", 3, 2 * G, 2, 128, 3000, kb, vb, g, 24, 6, 1900 + 10 * kb + G + g + window + block)
    pair = P.build_pair(w, L=3000, cap=3008)
    lens = np.array([2999, 777, 0])
    q = P.to_dev(pair["q"])
    k = 6 if block else 24
    st = DecodeStep(pair["lay"], k, 2999, window=window, block=block, exclude=True)
    out = st.attend(pair["gc"], q, lens)
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(w.B, w.Hq, 128)
    idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, st.row)
    orc = pair["oc"].decode(pair["q"], lens, st.row, sel=idx)
    P.assert_close(o, orc["out"], "exclude (window/blocks) vs oracle")


# INT8 query of the approximate scores (HACK review on Pith, Eq. (4)): every
# key width, both value widths, both GQA group sizes, groups of 32 and 64.
Q8_CASES = [(4, 4, 4, 32), (3, 2, 8, 32), (2, 2, 4, 64), (1, 2, 8, 64), (4, 2, 8, 64), (3, 4, 4, 32)]


@pytest.mark.parametrize("kb,vb,G,g", Q8_CASES)
def test_query_int8_step_parity(P, kb, vb, G, g):
    """Scores, selection and output against the oracle with qbits = 8."""
    banner(f"int8 query kb={kb} vb={vb} G={G} g={g}")
    w = P.Workload("q8", 2, 2 * G, 2, 128, 1000, kb, vb, g, 24, 6, 300 + 10 * kb + vb + G + g, query_bits=8)
    pair = P.build_pair(w, L=1000, cap=1024)
    lens = np.array([1000, 651])
    k = 24
    r = P.run_step(pair, lens, k)
    orc = pair["oc"].decode(pair["q"], lens, k, qbits=8)
    orc16 = pair["oc"].decode(pair["q"], lens, k)
    import oracle
    for b in range(w.B):
        n = lens[b]
        np.testing.assert_allclose(r["sigma"][b, :, :n], orc["sigma"][b, :, :n], rtol=1e-5, atol=2e-5)
        # the INT8 query moves the scores off the fp16-query ones
        assert not np.allclose(r["sigma"][b, :, :n], orc16["sigma"][b, :, :n], rtol=1e-6, atol=1e-7)
        for h in range(w.Hkv):
            want = oracle.topk(r["sigma"][b, h, :n].astype(np.float64), k)
            assert np.array_equal(r["idx"][b, h], want), (b, h)
            P.assert_topk_near_tie(r["idx"][b, h], orc["idx"][b, h], orc["sigma"][b, h], n, f"b{b}h{h}")
    orc_s = pair["oc"].decode(pair["q"], lens, k, sel=r["idx"], qbits=8)
    P.assert_close(r["out"], orc_s["out"], "out vs oracle(S_gpu)")
    P.assert_close(r["out"], orc["out"], "out vs oracle(S_oracle)")


@pytest.mark.parametrize("kb,vb,G,g", [(4, 4, 4, 32), (2, 2, 8, 64)])
def test_query_int8_decode_step_and_ends(P, kb, vb, G, g):
    """The one-launch step (append in the scan) with the INT8 query; k = 0 is
    the approximate output against the INT8 query, k = len the exact one."""
    import torch
    from bit_kv_attention_amd.step import DecodeStep
    banner(f"int8 query step/ends kb={kb} vb={vb} G={G} g={g}")
    w = P.Workload("q8s", 2, 2 * G, 2, 128, 900, kb, vb, g, 16, 4, 400 + kb + G, query_bits=8)
    pair = P.build_pair(w, L=900, cap=928)
    lens = np.array([900, 517])
    pos = [int(x) - 1 for x in lens]
    pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
    st = DecodeStep(pair["lay"], 16, 900)
    out = st.step(pair["gc"], P.to_dev(pair["q"]), P.to_dev(pair["k1"]), P.to_dev(pair["v1"]), pos)
    torch.cuda.synchronize()
    g_buf, o_buf = P.gpu_buffers(pair["gc"]), P.orc_buffers(pair["oc"])
    for name in g_buf:
        assert np.array_equal(g_buf[name], o_buf[name]), name
    got = out.cpu().numpy().reshape(w.B, w.Hq, 128)
    idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, 16)
    P.assert_close(got, pair["oc"].decode(pair["q"], lens, 16, sel=idx, qbits=8)["out"], "step vs oracle(S_gpu)")
    for k, key in ((0, "out_approx"), (900, "out_exact")):
        st2 = DecodeStep(pair["lay"], k, 900)
        o2 = st2.attend(pair["gc"], P.to_dev(pair["q"]), lens.tolist())
        torch.cuda.synchronize()
        ref = pair["oc"].decode(pair["q"], lens, k, want_approx=True, want_exact=True, qbits=8)
        P.assert_close(o2.cpu().numpy().reshape(w.B, w.Hq, 128), ref[key], f"k={k}")


# MXFP4 keys (E2M1 codes, one power-of-two scale per group of 32): both value
# widths and both GQA group sizes, for key format 2 (E8M0 scales, scores
# against the MXFP4 query on the scaled FP4 MFMA) and key format 1 (fp16
# scales, scores against the fp16 query).
MX_CASES = [(4, 4, 2), (2, 8, 2), (4, 8, 2), (2, 4, 2), (4, 4, 1), (2, 8, 1), (4, 8, 1), (2, 4, 1)]


@pytest.mark.parametrize("vb,G,kf", MX_CASES)
def test_mxfp4_keys_step_parity(P, vb, G, kf):
    """Pack bit-exact, then scores, selection and output against the oracle
    with MXFP4 keys."""
    banner(f"mxfp4 keys vb={vb} G={G} key format {kf}")
    import oracle
    w = P.Workload("mx", 2, 2 * G, 2, 128, 1000, 4, vb, 32, 24, 6, 500 + vb + G, key_format=kf)
    pair = P.build_pair(w, L=1000, cap=1024)
    lens = np.array([1000, 651])
    k = 24
    r = P.run_step(pair, lens, k)
    g_buf, o_buf = P.gpu_buffers(pair["gc"]), P.orc_buffers(pair["oc"])
    for name in g_buf:
        assert np.array_equal(g_buf[name], o_buf[name]), name
    orc = pair["oc"].decode(pair["q"], lens, k)
    for b in range(w.B):
        n = lens[b]
        np.testing.assert_allclose(r["sigma"][b, :, :n], orc["sigma"][b, :, :n], rtol=1e-5, atol=2e-5)
        for h in range(w.Hkv):
            want = oracle.topk(r["sigma"][b, h, :n].astype(np.float64), k)
            assert np.array_equal(r["idx"][b, h], want), (b, h)
            P.assert_topk_near_tie(r["idx"][b, h], orc["idx"][b, h], orc["sigma"][b, h], n, f"b{b}h{h}")
    orc_s = pair["oc"].decode(pair["q"], lens, k, sel=r["idx"])
    P.assert_close(r["out"], orc_s["out"], "out vs oracle(S_gpu)")
    P.assert_close(r["out"], orc["out"], "out vs oracle(S_oracle)")


@pytest.mark.parametrize("vb,G,kf", [(4, 4, 2), (2, 8, 2), (4, 8, 1), (2, 4, 1)])
def test_mxfp4_keys_decode_step_and_ends(P, vb, G, kf):
    """The one-launch step (MXFP4 append inside the scan), then k = 0 (the
    approximate output over the MXFP4 keys) and k = len (exact)."""
    import torch
    from bit_kv_attention_amd.step import DecodeStep
    banner(f"mxfp4 keys step/ends vb={vb} G={G} key format {kf}")
    w = P.Workload("mxs", 2, 2 * G, 2, 128, 900, 4, vb, 32, 16, 4, 600 + vb + G, key_format=kf)
    pair = P.build_pair(w, L=900, cap=928)
    lens = np.array([900, 517])
    pos = [int(x) - 1 for x in lens]
    pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
    st = DecodeStep(pair["lay"], 16, 900)
    out = st.step(pair["gc"], P.to_dev(pair["q"]), P.to_dev(pair["k1"]), P.to_dev(pair["v1"]), pos)
    torch.cuda.synchronize()
    g_buf, o_buf = P.gpu_buffers(pair["gc"]), P.orc_buffers(pair["oc"])
    for name in g_buf:
        assert np.array_equal(g_buf[name], o_buf[name]), name
    got = out.cpu().numpy().reshape(w.B, w.Hq, 128)
    idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, 16)
    P.assert_close(got, pair["oc"].decode(pair["q"], lens, 16, sel=idx)["out"], "step vs oracle(S_gpu)")
    for k, key in ((0, "out_approx"), (900, "out_exact")):
        st2 = DecodeStep(pair["lay"], k, 900)
        o2 = st2.attend(pair["gc"], P.to_dev(pair["q"]), lens.tolist())
        torch.cuda.synchronize()
        ref = pair["oc"].decode(pair["q"], lens, k, want_approx=True, want_exact=True)
        P.assert_close(o2.cpu().numpy().reshape(w.B, w.Hq, 128), ref[key], f"k={k}")
