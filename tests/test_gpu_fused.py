"""GPU parity of the fused step (qattn_decode_fused: append, scan, top-k and
correction in one launch) against the oracle and against the same step run
as separate launches.

sigma and idx must be identical to the separate launches' (same scan code,
same selection definition); the output must meet the oracle tolerance on the
GPU's own selected set and on the oracle's.  Every case also checks that no
unit barrier gave up waiting (the flag word of the workspace)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

COMBOS = [(kb, vb, G) for kb in (4, 3) for vb in (4, 2) for G in (4, 8)]


@pytest.fixture(scope="module")
def P(orc):
    import parity
    return parity


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def flag_word(st, lay):
    """Bit 0 set = a unit barrier of the fused step stopped waiting."""
    units = lay.batch * lay.n_kv_heads
    off = ((units * 4 + 255) // 256) * 256 + units * 8
    return int(st.ws.cpu().numpy().view(np.uint32)[off // 4])


def fused_and_separate(P, lay, k, max_len):
    from bit_kv_attention_amd.step import DecodeStep
    a = DecodeStep(lay, k, max_len, one_launch=True)
    b = DecodeStep(lay, k, max_len, one_launch=False)
    assert a.one_launch and not b.one_launch
    return a, b


def check_against_oracle(P, pair, r, lens, k):
    import oracle
    w = pair["w"]
    orc = pair["oc"].decode(pair["q"], lens, k)
    for b in range(w.B):
        for h in range(w.Hkv):
            n = int(lens[b])
            if n == 0:
                assert np.all(r["idx"][b, h] == -1)
                continue
            want = oracle.topk(r["sigma"][b, h, :n].astype(np.float64), k)
            assert np.array_equal(r["idx"][b, h], want), (b, h)
            P.assert_topk_near_tie(r["idx"][b, h], orc["idx"][b, h], orc["sigma"][b, h], n, f"b{b}h{h}")
    orc_s = pair["oc"].decode(pair["q"], lens, k, sel=np.where(r["idx"] < 0, -1, r["idx"]))
    e1 = P.assert_close(r["out"], orc_s["out"], "fused out vs oracle(S_gpu)")
    e2 = P.assert_close(r["out"], orc["out"], "fused out vs oracle(S_oracle)")
    return max(e1, e2)


def run_both(P, pair, lens, k, append=True):
    """The step (append of the pair's new token at lens-1, then attention over
    lens) through the fused launch and through the separate launches, on two
    caches holding the same tokens.  Returns both results as numpy."""
    import torch
    from bit_kv_attention_amd import binding as bk
    w = pair["w"]
    lay = pair["lay"]
    gc2 = bk.allocate_cache(lay)
    for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow"):
        getattr(gc2, name).copy_(getattr(pair["gc"], name))
    pos = [max(int(x) - 1, 0) for x in lens]
    a, b = fused_and_separate(P, lay, k, int(max(lens)))
    q = P.to_dev(pair["q"])
    kn, vn = P.to_dev(pair["k1"]), P.to_dev(pair["v1"])
    if append:
        pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
        a.step(pair["gc"], q, kn, vn, pos)
        b.step(gc2, q, kn, vn, pos)
    else:
        a.attend(pair["gc"], q, lens)
        b.attend(gc2, q, lens)
    torch.cuda.synchronize()
    assert a.ran_fused, "the fused step fell back to the separate launches"
    cap = pair["cap"]
    res = []
    for st in (a, b):
        res.append(dict(out=st.out.cpu().numpy().reshape(w.B, w.Hq, 128),
                        sigma=st.sigma.cpu().numpy().reshape(w.B, w.Hkv, cap),
                        idx=st.idx.cpu().numpy().reshape(w.B, w.Hkv, max(k, 1))[:, :, :k]))
    if append:
        ga, gb = P.gpu_buffers(pair["gc"]), P.gpu_buffers(gc2)
        for name in ga:
            assert np.array_equal(ga[name], gb[name]), name
    assert flag_word(a, lay) == 0
    return res


def assert_same_selection(ra, rb, lens):
    for b in range(len(lens)):
        n = int(lens[b])
        assert np.array_equal(ra["sigma"][b, :, :n], rb["sigma"][b, :, :n]), b
    assert np.array_equal(ra["idx"], rb["idx"])


@pytest.mark.parametrize("kb,vb,G", COMBOS)
def test_fused_step_parity(P, kb, vb, G):
    """Ragged lengths over several splits; the append inside the launch."""
    banner(f"fused step kb={kb} vb={vb} G={G}")
    w = P.Workload("fused", 3, 2 * G, 2, 128, 5000, kb, vb, 32, 40, 8, 300 + 10 * kb + vb + G)
    pair = P.build_pair(w, L=5000, cap=5024)
    lens = np.array([5000, 2311, 777])
    ra, rb = run_both(P, pair, lens, w.k)
    assert_same_selection(ra, rb, lens)
    check_against_oracle(P, pair, ra, lens, w.k)
    check_against_oracle(P, pair, rb, lens, w.k)


@pytest.mark.parametrize("kb,vb,G", [(4, 4, 4), (3, 2, 8)])
def test_fused_step_crowded_selection(P, kb, vb, G):
    """Selected tokens crowded into the first split (their keys follow the
    query), so that one workgroup corrects several passes of them while
    others correct few or none.  Ragged lengths; every sequence appends."""
    banner(f"fused step, crowded selection kb={kb} vb={vb} G={G}")
    w = P.Workload("crowded", 3, 2 * G, 2, 128, 5000, kb, vb, 32, 300, 8, 500 + 10 * kb + vb + G)

    def crowd(inp):  # tokens 0..399 of each (b, kvh): keys along the group's first query head, plus noise
        rng = np.random.default_rng(7)
        for b in range(w.B):
            for h in range(w.Hkv):
                qd = inp.q[b, h * G].astype(np.float32)
                noise = rng.standard_normal((400, 128)).astype(np.float32)
                inp.K[b, h, :400] = (0.5 * qd[None, :] + 0.3 * noise).astype(np.float16)

    pair = P.build_pair(w, L=5000, cap=5024, tweak=crowd)
    lens = np.array([5000, 2311, 777])
    ra, rb = run_both(P, pair, lens, w.k)
    # the crowding worked: more than a pass of selected tokens in the first split
    assert all(int((ra["idx"][b, h] < 256).sum()) > 64 for b in range(w.B) for h in range(w.Hkv))
    assert_same_selection(ra, rb, lens)
    check_against_oracle(P, pair, ra, lens, w.k)


@pytest.mark.parametrize("kf,vb,G", [(2, 4, 4), (2, 2, 8), (1, 4, 4), (1, 2, 8)])
def test_fused_step_parity_mxfp4(P, kf, vb, G):
    """MXFP4 keys in the fused launch: key format 2 (scores FP4 x FP4 on the
    scaled MFMA, the correction's approximate logits from the same FP4 query)
    and key format 1 (fp16 query); ragged lengths, the append inside."""
    banner(f"fused step mxfp4 kf={kf} vb={vb} G={G}")
    w = P.Workload("fusedmx", 3, 2 * G, 2, 128, 5000, 4, vb, 32, 40, 8, 600 + 10 * kf + vb + G, key_format=kf)
    pair = P.build_pair(w, L=5000, cap=5024)
    lens = np.array([5000, 2311, 777])
    ra, rb = run_both(P, pair, lens, w.k)
    assert_same_selection(ra, rb, lens)
    check_against_oracle(P, pair, ra, lens, w.k)
    check_against_oracle(P, pair, rb, lens, w.k)


@pytest.mark.parametrize("kb,vb,G", [(4, 4, 4), (3, 2, 8)])
def test_fused_many_selected_per_split(P, kb, vb, G):
    """k far above 64 per split (about 128 selected tokens in each split of
    512): most selected tokens lie outside each split's likely set and take
    passes of their own after the threshold."""
    banner(f"fused many per split kb={kb} vb={vb} G={G}")
    w = P.Workload("fmany", 4, 8 * G, 8, 128, 4096, kb, vb, 32, 1024, 8, 500 + kb + G)
    pair = P.build_pair(w, L=4096, cap=4096)
    lens = np.array([4096, 4000, 3001, 2048])
    ra, rb = run_both(P, pair, lens, w.k)
    assert_same_selection(ra, rb, lens)
    check_against_oracle(P, pair, ra, lens, w.k)


@pytest.mark.parametrize("kb,vb,G", [(4, 4, 4), (3, 2, 8)])
def test_fused_attend_without_append(P, kb, vb, G):
    banner(f"fused attend kb={kb} vb={vb} G={G}")
    w = P.Workload("fattend", 2, 4 * G, 4, 128, 3000, kb, vb, 32, 64, 10, 400 + kb + G)
    pair = P.build_pair(w, L=3000, cap=3008)
    lens = np.array([2999, 1500])
    pos = [int(x) - 1 for x in lens]
    from bit_kv_attention_amd import binding as bk
    bk.kv_pack_append(pair["lay"], pair["gc"], P.to_dev(pair["k1"]), P.to_dev(pair["v1"]), 1, pos)
    pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
    ra, rb = run_both(P, pair, lens, w.k, append=False)
    assert_same_selection(ra, rb, lens)
    check_against_oracle(P, pair, ra, lens, w.k)


def test_fused_edge_lengths(P):
    """len 0, 1, 31, 33 and one long ragged sequence in one batch (empty
    splits, a unit with nothing to select, units with k > len)."""
    banner("fused edge lengths")
    w = P.Workload("fedge", 5, 8, 2, 128, 1100, 3, 2, 32, 16, 2, 56)
    pair = P.build_pair(w, L=1100, cap=1120)
    lens = np.array([0, 1, 31, 33, 1100])
    from bit_kv_attention_amd import binding as bk
    # the new token at lens - 1 by a separate append (a length of 0 has no slot)
    pos = [max(int(x) - 1, 0) for x in lens]
    bk.kv_pack_append(pair["lay"], pair["gc"], P.to_dev(pair["k1"]), P.to_dev(pair["v1"]), 1, pos)
    pair["oc"].append(pair["k1"], pair["v1"], np.array(pos, np.int32))
    ra, rb = run_both(P, pair, lens, w.k, append=False)
    assert_same_selection(ra, rb, lens)
    assert np.all(ra["out"][0] == 0)
    assert np.all(ra["idx"][0] == -1)
    check_against_oracle(P, pair, ra, lens, w.k)


@pytest.mark.parametrize("k", [0, 700, 2000])
def test_fused_approx_only_and_exact(P, k):
    """k = 0: the approximate output; k >= len: exact attention (every split
    keeps only its exact state)."""
    banner(f"fused k={k}")
    import torch
    from bit_kv_attention_amd.step import DecodeStep
    w = P.Workload("fends", 2, 8, 2, 128, 700, 4, 4, 32, 0, 4, 71)
    pair = P.build_pair(w, L=700, cap=704)
    lens = np.array([700, 333])
    st = DecodeStep(pair["lay"], k, 700, one_launch=True)
    assert st.one_launch
    out = st.attend(pair["gc"], P.to_dev(pair["q"]), lens)
    torch.cuda.synchronize()
    orc = pair["oc"].decode(pair["q"], lens, 0, want_approx=True, want_exact=True)
    ref = orc["out_approx"] if k == 0 else orc["out_exact"]
    P.assert_close(out.cpu().numpy().reshape(w.B, w.Hq, 128), ref, f"k={k}")
    if k:
        idx = st.idx.cpu().numpy().reshape(w.B, w.Hkv, k)
        for b in range(w.B):
            assert idx[b, :, :lens[b]].tolist() == [list(range(lens[b]))] * w.Hkv
            assert np.all(idx[b, :, lens[b]:] == -1)
    assert flag_word(st, pair["lay"]) == 0


@pytest.mark.parametrize("L,k", [(10000, 50), (3000, 257)])
def test_fused_ties_overflow(P, L, k):
    """All keys equal (one clear winner): every score falls in one histogram
    bin, each split holds more of them than its list, so the threshold comes
    from the radix select over sigma; the set is the lowest indices."""
    banner(f"fused ties L={L} k={k}")
    import torch
    import oracle
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    rng = np.random.default_rng(9)
    cap = ((L + 31) // 32) * 32
    row = rng.standard_normal(128).astype(np.float16)
    K = np.tile(row, (1, 1, L, 1))
    K[0, 0, L // 3] = (row.astype(np.float32) * 2).astype(np.float16)
    V = rng.standard_normal((1, 1, L, 128)).astype(np.float16)
    q = rng.standard_normal((1, 4, 128)).astype(np.float16)
    lay = bk.make_layout(1, 4, 1, cap, 4, 4)
    gc = bk.allocate_cache(lay)
    bk.kv_pack_append(lay, gc, P.to_dev(K), P.to_dev(V), L, [0])
    st = DecodeStep(lay, k, L, one_launch=True)
    assert st.one_launch
    out = st.attend(gc, P.to_dev(q), [L])
    torch.cuda.synchronize()
    sig = st.sigma.cpu().numpy()[:L].astype(np.float64)
    idx = st.idx.cpu().numpy()[:k]
    assert np.array_equal(idx, oracle.topk(sig, k))
    oc = oracle.Cache(oracle.Shape(1, 4, 1, 128, 4, 4, 32, cap))
    oc.append(K, V, np.zeros(1, np.int32))
    ref = oc.decode(q, np.array([L], np.int32), k, sel=idx.reshape(1, 1, -1))
    P.assert_close(out.cpu().numpy().reshape(1, 4, 128), ref["out"], "ties out")
    assert flag_word(st, lay) == 0


def test_fused_tie_group_at_threshold(P):
    """A few equal scores straddle the threshold in different splits: the
    threshold lies inside a group whose composites share every score bit, so
    it is found by ranking the group's entries (the lower indices win)."""
    banner("fused tie group at the threshold")
    import torch
    import oracle
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    rng = np.random.default_rng(21)
    L, k = 4000, 5
    cap = ((L + 31) // 32) * 32
    q = rng.standard_normal((1, 4, 128)).astype(np.float16)
    K = rng.standard_normal((1, 1, L, 128)).astype(np.float16)
    d = q[0, 0].astype(np.float32) / np.linalg.norm(q[0, 0].astype(np.float32))
    for t, s in ((50, 2.5), (2000, 2.0), (3500, 1.5)):  # three clear winners
        K[0, 0, t] = (d * 12 * s).astype(np.float16)
    for t in (3900, 100, 2500, 1500, 3000):  # the tied group: two of them are taken
        K[0, 0, t] = (d * 12).astype(np.float16)
    V = rng.standard_normal((1, 1, L, 128)).astype(np.float16)
    lay = bk.make_layout(1, 4, 1, cap, 4, 4)
    gc = bk.allocate_cache(lay)
    bk.kv_pack_append(lay, gc, P.to_dev(K), P.to_dev(V), L, [0])
    st = DecodeStep(lay, k, L, one_launch=True)
    assert st.one_launch
    out = st.attend(gc, P.to_dev(q), [L])
    torch.cuda.synchronize()
    sig = st.sigma.cpu().numpy()[:L].astype(np.float64)
    idx = st.idx.cpu().numpy()[:k]
    assert sig[100] == sig[1500] == sig[2500] == sig[3000] == sig[3900]
    assert np.array_equal(idx, oracle.topk(sig, k))
    assert set(idx.tolist()) == {50, 100, 1500, 2000, 3500}
    oc = oracle.Cache(oracle.Shape(1, 4, 1, 128, 4, 4, 32, cap))
    oc.append(K, V, np.zeros(1, np.int32))
    ref = oc.decode(q, np.array([L], np.int32), k, sel=idx.reshape(1, 1, -1))
    P.assert_close(out.cpu().numpy().reshape(1, 4, 128), ref["out"], "tie group out")
    assert flag_word(st, lay) == 0


def test_fused_repeated_steps(P):
    """Four steps in a row on one workspace (counters and histograms back at
    zero after each), lengths growing by one, against the separate launches."""
    banner("fused repeated steps")
    import torch
    from bit_kv_attention_amd import binding as bk
    w = P.Workload("frep", 4, 32, 8, 128, 8192, 4, 4, 32, 128, 16, 77)
    inp = P.make_inputs(w, L=8000)
    lay = bk.make_layout(w.B, w.Hq, w.Hkv, 8192, 4, 4)
    caches = [bk.allocate_cache(lay) for _ in range(2)]
    for c in caches:
        bk.kv_pack_append(lay, c, P.to_dev(inp.K), P.to_dev(inp.V), 8000, [0] * w.B)
    knew, vnew = P.make_new_tokens(w, 4, inp.outlier_ch)
    a, b = fused_and_separate(P, lay, w.k, 8192)
    q = P.to_dev(inp.q)
    for i in range(4):
        pos = [8000 + i] * w.B
        kn, vn = P.to_dev(knew[i]), P.to_dev(vnew[i])
        a.step(caches[0], q, kn, vn, pos)
        b.step(caches[1], q, kn, vn, pos)
        torch.cuda.synchronize()
        assert torch.equal(a.idx, b.idx), i
        sa = a.sigma.reshape(w.B * w.Hkv, -1)[:, :8001 + i]
        sb = b.sigma.reshape(w.B * w.Hkv, -1)[:, :8001 + i]
        assert torch.equal(sa, sb), i
        P.assert_close(a.out.cpu().numpy(), b.out.cpu().numpy(), f"step {i}")
        assert flag_word(a, lay) == 0
