"""Pins of the oracle's scores, selection and corrected output (O3-O5).

Approximate-then-correct (JetFire README, introduction): attention over the
dequantised low-bit cache, with the top-k tokens' logits and values replaced by
exact ones.  Pinned against independent fp64 numpy computations: dense softmax
attention (k >= L reduces to it exactly), attention over the dequantised cache
(k = 0), the GQA/MHA equivalence, closed forms, invariances, brute-force top-k,
and the HACK Eq. (4) identity the GPU kernels rely on.
"""
import numpy as np
import pytest

from bit_kv_attention_amd.synth import Workload, make_inputs


def small_workload(**kw):
    base = dict(name="t", B=2, Hq=8, Hkv=2, D=128, L=300, kbits=4, vbits=4, group=32,
                k=12, planted=6, seed=77)
    base.update(kw)
    return Workload(**base)


def build(orc, w, inp, cap=None):
    cap = cap or ((w.L + 31) // 32) * 32
    s = orc.Shape(w.B, w.Hq, w.Hkv, w.D, w.kbits, w.vbits, w.group, cap)
    cache = orc.Cache(s)
    cache.append(inp.K, inp.V, np.zeros(w.B, np.int32))
    return cache


def dense(q, K, V, G):
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            s = K[b, h // G] @ q[b, h] / np.sqrt(D)
            p = np.exp(s - s.max())
            out[b, h] = p @ V[b, h // G] / p.sum()
    return out


def dequant_np(orc, X, g, bits):
    codes, s16, z16 = orc.quantize_rows(X, g, bits)
    s = np.repeat(s16.view(np.float16).astype(np.float64), g, axis=-1)
    z = np.repeat(z16.view(np.float16).astype(np.float64), g, axis=-1)
    return s * codes + z


@pytest.mark.parametrize("kb,vb,g", [(4, 4, 32), (3, 2, 32), (2, 2, 64), (1, 2, 64)])
def test_k_all_equals_dense_fp16_attention(orc, kb, vb, g):
    w = small_workload(kbits=kb, vbits=vb, group=g)
    inp = make_inputs(w)
    cache = build(orc, w, inp)
    lens = np.full(w.B, w.L)
    r = cache.decode(inp.q, lens, k=w.L, want_exact=True)
    ref = dense(inp.q.astype(np.float64), inp.K.astype(np.float64), inp.V.astype(np.float64), w.G)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["out_exact"], ref, rtol=1e-11, atol=1e-12)
    r2 = cache.decode(inp.q, lens, k=10 * w.L)  # k > L selects everything
    np.testing.assert_allclose(r2["out"], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("kb,vb,g", [(4, 4, 32), (3, 2, 32), (4, 2, 32), (3, 4, 32), (2, 2, 32), (1, 4, 32),
                                     (4, 4, 64), (2, 2, 64), (1, 2, 64)])
def test_k_zero_equals_attention_over_dequantised_cache(orc, kb, vb, g):
    w = small_workload(kbits=kb, vbits=vb, group=g)
    inp = make_inputs(w)
    cache = build(orc, w, inp)
    r = cache.decode(inp.q, np.full(w.B, w.L), k=0, want_approx=True)
    Kh = dequant_np(orc, inp.K, g, kb)
    Vh = dequant_np(orc, inp.V, g, vb)
    ref = dense(inp.q.astype(np.float64), Kh, Vh, w.G)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["out_approx"], ref, rtol=1e-11, atol=1e-12)
    # sigma = max over the group's heads of the approximate logit
    for b in range(w.B):
        for kvh in range(w.Hkv):
            sh = np.stack([Kh[b, kvh] @ inp.q[b, h].astype(np.float64) / np.sqrt(w.D)
                           for h in range(kvh * w.G, (kvh + 1) * w.G)])
            np.testing.assert_allclose(r["sigma"][b, kvh, :w.L], sh.max(0), rtol=1e-12, atol=1e-12)


def test_selected_tokens_use_exact_logits_and_values(orc):
    """O5 for a given set equals the mixture computed directly in numpy."""
    w = small_workload(kbits=3, vbits=2, L=200)
    inp = make_inputs(w)
    cache = build(orc, w, inp)
    rng = np.random.default_rng(4)
    k = 17
    sel = np.stack([[np.sort(rng.choice(w.L, k, replace=False)) for _ in range(w.Hkv)] for _ in range(w.B)])
    r = cache.decode(inp.q, np.full(w.B, w.L), k=k, sel=sel)
    Kh = dequant_np(orc, inp.K, 32, 3)
    Vh = dequant_np(orc, inp.V, 32, 2)
    K = inp.K.astype(np.float64)
    V = inp.V.astype(np.float64)
    for b in range(w.B):
        for h in range(w.Hq):
            kvh = h // w.G
            m = np.zeros(w.L, bool)
            m[sel[b, kvh]] = True
            q = inp.q[b, h].astype(np.float64)
            lam = np.where(m, K[b, kvh] @ q, Kh[b, kvh] @ q) / np.sqrt(w.D)
            nu = np.where(m[:, None], V[b, kvh], Vh[b, kvh])
            p = np.exp(lam - lam.max())
            np.testing.assert_allclose(r["out"][b, h], p @ nu / p.sum(), rtol=1e-11, atol=1e-12)


def test_gqa_equals_replicated_mha(orc):
    w = small_workload(B=1, Hq=8, Hkv=2, L=150)
    inp = make_inputs(w)
    g = build(orc, w, inp)
    wm = w.with_(Hkv=8)
    Kr = np.repeat(inp.K, 4, axis=1)
    Vr = np.repeat(inp.V, 4, axis=1)
    s = orc.Shape(1, 8, 8, 128, w.kbits, w.vbits, 32, 160)
    m = orc.Cache(s)
    m.append(Kr, Vr, [0])
    for k in (0, w.L):
        a = g.decode(inp.q, [w.L], k=k)["out"]
        b = m.decode(inp.q, [w.L], k=k)["out"]
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_equal_keys_give_mean_value(orc):
    rng = np.random.default_rng(2)
    L = 100
    K = np.tile(rng.standard_normal((1, 1, 1, 128)), (1, 1, L, 1)).astype(np.float16)
    V = rng.standard_normal((1, 1, L, 128)).astype(np.float16)
    q = rng.standard_normal((1, 4, 128)).astype(np.float16)
    s = orc.Shape(1, 4, 1, 128, 4, 2, 32, 128)
    c = orc.Cache(s)
    c.append(K, V, [0])
    Vh = dequant_np(orc, V, 32, 2)
    np.testing.assert_allclose(c.decode(q, [L], k=0)["out"][0], np.tile(Vh[0, 0].mean(0), (4, 1)), rtol=1e-12)
    np.testing.assert_allclose(c.decode(q, [L], k=L)["out"][0],
                               np.tile(V[0, 0].astype(np.float64).mean(0), (4, 1)), rtol=1e-12)


def test_token_permutation_invariance(orc):
    w = small_workload(B=1, Hq=4, Hkv=1, L=128, planted=0)
    inp = make_inputs(w)
    perm = np.random.default_rng(3).permutation(w.L)
    a = build(orc, w, inp)
    inp2 = type(inp)(q=inp.q, K=inp.K[:, :, perm], V=inp.V[:, :, perm], outlier_ch=inp.outlier_ch,
                     planted_pos=inp.planted_pos)
    b = build(orc, w, inp2)
    for k in (0, 9, w.L):
        ra = a.decode(inp.q, [w.L], k=k)
        rb = b.decode(inp.q, [w.L], k=k)
        np.testing.assert_allclose(ra["out"], rb["out"], rtol=1e-12, atol=1e-13)
        if 0 < k < w.L:
            assert sorted(perm[rb["idx"][0, 0]].tolist()) == ra["idx"][0, 0].tolist()


def test_topk_brute_force_and_ties(orc):
    rng = np.random.default_rng(8)
    for n in (0, 1, 5, 40, 257):
        sig = np.round(rng.standard_normal(n) * 3) / 2  # many exact ties
        for k in (0, 1, 3, 16, n, n + 5):
            got = orc.topk(sig, k)
            order = sorted(range(n), key=lambda t: (-sig[t], t))
            want = sorted(order[:min(k, n)]) + [-1] * (k - min(k, n))
            assert got.tolist() == want


def test_planted_tokens_are_selected(orc):
    """The needle analogue: every planted token (cosine 0.9 with one query of
    the group) is in the selected set."""
    w = Workload("tiny", 1, 4, 1, 128, 1024, 4, 4, 32, 16, 8, 1000)
    inp = make_inputs(w)
    cache = build(orc, w, inp)
    r = cache.decode(inp.q, [w.L], k=w.k)
    assert set(inp.planted_pos[0, 0].tolist()) <= set(r["idx"][0, 0].tolist())


def test_ragged_lengths_and_empty(orc):
    w = small_workload(B=3, Hq=4, Hkv=1, L=96)
    inp = make_inputs(w)
    cache = build(orc, w, inp)
    lens = np.array([96, 37, 0])
    r = cache.decode(inp.q, lens, k=8, want_exact=True)
    assert np.all(r["out"][2] == 0)
    assert np.all(r["idx"][2] == -1)
    ref = dense(inp.q[1:2].astype(np.float64), inp.K[1:2, :, :37].astype(np.float64),
                inp.V[1:2, :, :37].astype(np.float64), 4)
    np.testing.assert_allclose(r["out_exact"][1:2], ref, rtol=1e-11)


def test_hack_eq4_identity_for_unquantised_query():
    """HACK review on Pith, Eq. (4): with x_hat = s*c + z per group and an
    unquantised q, q . x_hat = s * (q . c) + z * sum(q).  Exact in fp64; in fp32
    the two forms agree to fp32 rounding.  The GPU score path uses the
    right-hand form."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        q = rng.standard_normal(32).astype(np.float16).astype(np.float64)
        c = rng.integers(0, 16, 32).astype(np.float64)
        s = float(np.float16(abs(rng.standard_normal()) / 4))
        z = float(np.float16(rng.standard_normal()))
        lhs = q @ (s * c + z)
        rhs = s * (q @ c) + z * q.sum()
        assert abs(lhs - rhs) <= 1e-12 * (np.abs(q) @ np.abs(s * c + z) + 1)
        q32, c32 = q.astype(np.float32), c.astype(np.float32)
        rhs32 = np.float32(s) * (q32 @ c32) + np.float32(z) * q32.sum(dtype=np.float32)
        assert abs(float(rhs32) - lhs) <= 4e-6 * (np.abs(q) @ np.abs(s * c + z) + abs(z) * np.abs(q).sum())


def test_topk_window_brute_force(orc):
    """O4 with a recent window: the last min(w, n) tokens always, plus the k
    largest (ties to the lower index) of the tokens before them; ascending,
    then -1.  w = 0 is plain O4; w >= n selects every token."""
    rng = np.random.default_rng(11)
    for n in (0, 1, 7, 40, 130):
        sig = np.round(rng.standard_normal(n) * 3) / 2  # many exact ties
        for k in (0, 1, 5, n, n + 3):
            for w in (0, 1, 4, n, n + 2):
                got = orc.topk_window(sig, k, w)
                nw = min(w, n)
                n0 = n - nw
                order = sorted(range(n0), key=lambda t: (-sig[t], t))
                want = sorted(order[:min(k, n0)]) + list(range(n0, n))
                want += [-1] * (k + w - len(want))
                assert got.tolist() == want, (n, k, w)
                if w == 0:
                    assert got.tolist() == orc.topk(sig, k).tolist()


def test_window_covering_everything_equals_dense_attention(orc):
    """A window as long as the context puts every token in the exact set: the
    corrected output is then dense fp16 attention, even with k = 0."""
    w = small_workload(kbits=3, vbits=2, L=120)
    inp = make_inputs(w)
    cache = build(orc, w, inp)
    lens = np.full(w.B, w.L)
    r0 = cache.decode(inp.q, lens, k=0, want_approx=True)
    win = w.L
    sel = np.stack([[orc.topk_window(r0["sigma"][b, h, :w.L], 0, win) for h in range(w.Hkv)]
                    for b in range(w.B)])
    r = cache.decode(inp.q, lens, k=win, sel=sel)
    ref = dense(inp.q.astype(np.float64), inp.K.astype(np.float64), inp.V.astype(np.float64), w.G)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)


def test_topk_blocks_brute_force(orc):
    """O4 by blocks: every chosen block beats every other block by (largest
    sigma desc, block index asc), the blocks come out ascending as their
    tokens (the ragged last one cut at n), then -1; block size 1 is plain
    O4, and a budget covering every block lists every token."""
    rng = np.random.default_rng(12)
    for n in (0, 1, 7, 40, 131):
        sig = np.round(rng.standard_normal(n) * 3) / 2  # many exact ties
        for bs in (1, 2, 4, 32):
            nblk = -(-n // bs)
            score = [max(sig[j * bs:(j + 1) * bs]) for j in range(nblk)]
            for nb in (0, 1, 3, nblk, nblk + 2):
                got = orc.topk_blocks(sig, nb, bs)
                assert got.shape == (nb * bs,)
                kb = min(nb, nblk)
                chosen = [int(got[r * bs]) // bs for r in range(kb)]
                assert chosen == sorted(set(chosen)) and len(chosen) == kb, (n, bs, nb)
                for c in chosen:
                    for j in set(range(nblk)) - set(chosen):
                        assert score[c] > score[j] or (score[c] == score[j] and c < j), (n, bs, nb, c, j)
                want = [t for c in chosen for t in list(range(c * bs, min(n, c * bs + bs))) +
                        [-1] * (c * bs + bs - min(n, c * bs + bs))]
                want += [-1] * (nb * bs - len(want))
                assert got.tolist() == want, (n, bs, nb)
                if bs == 1:
                    assert got.tolist() == orc.topk(sig, nb).tolist()
                if nb >= nblk:
                    assert got[:n].tolist() == list(range(n))


def test_topk_blocks_planted_token_selects_its_block(orc):
    """One token far above the rest puts its block first; with one block of
    budget exactly that block is listed."""
    rng = np.random.default_rng(13)
    sig = rng.standard_normal(1000)
    for t in (0, 127, 128, 517, 999):
        s = sig.copy()
        s[t] = 50.0
        got = orc.topk_blocks(s, 1, 128)
        j = t // 128
        want = list(range(j * 128, min(1000, j * 128 + 128)))
        assert got.tolist() == want + [-1] * (128 - len(want)), t


def test_blocks_covering_everything_equals_dense_attention(orc):
    """A block budget covering the context corrects every token: the output
    is dense fp16 attention."""
    w = small_workload(kbits=4, vbits=4, L=120)
    inp = make_inputs(w)
    cache = build(orc, w, inp)
    lens = np.full(w.B, w.L)
    r0 = cache.decode(inp.q, lens, k=0, want_approx=True)
    nb, bs = 4, 32
    sel = np.stack([[orc.topk_blocks(r0["sigma"][b, h, :w.L], nb, bs) for h in range(w.Hkv)]
                    for b in range(w.B)])
    r = cache.decode(inp.q, lens, k=nb * bs, sel=sel)
    ref = dense(inp.q.astype(np.float64), inp.K.astype(np.float64), inp.V.astype(np.float64), w.G)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)
