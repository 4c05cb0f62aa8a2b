"""Pins of the oracle's key format 2: MXFP4 keys with E8M0 scales and an
MXFP4 query, i.e. FP4 query-key scores (Jet-QSparse abstract: FP4 keys and a
native FP4 query-key product; the OCP Microscaling formats define the block:
32 E2M1 elements sharing one scale 2^X, X = floor(log2(amax)) - 2, stored as
the E8M0 byte X + 127).

Pinned by hand-derived blocks, brute force over the E2M1 grid, the layout
restated as the lane operands of a 16x16x128 FP4 matrix product, inputs that
lie on the MX grid (quantisation is then exact, so the approximate scores
must equal the plain fp64 dot products), and attention computed in numpy from
the codes.
"""
import numpy as np
import pytest

from bit_kv_attention_amd.synth import Workload, make_inputs

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _val(code):
    return (-1.0 if code & 8 else 1.0) * E2M1[code & 7]


def _dequant(codes, e8):
    """E2M1 values times 2^(e8 - 127) per 32-channel block (numpy, fp64)."""
    vals = np.vectorize(_val)(codes.astype(np.int64))
    return vals * np.repeat(np.ldexp(1.0, e8.astype(np.int64) - 127), 32, axis=-1)


def test_hand_derived_block(orc):
    """amax = 1.0, so X = 0 - 2: byte 125, scale 0.25; (x, expected code)."""
    cases = [(1.0, 6), (-1.0, 14), (0.3125, 2), (0.4375, 4), (0.0625, 0), (0.875, 6), (0.625, 4),
             (0.1875, 2), (0.7, 5), (-0.01, 0), (0.125, 1), (-0.375, 11)]
    x = np.zeros(32, dtype=np.float16)
    for i, (v, _) in enumerate(cases):
        x[i] = v
    codes, e8 = orc.quantize_rows_mx8(x[None])
    assert e8[0, 0] == 125
    assert [int(c) for c in codes[0, :len(cases)]] == [c for _, c in cases]
    assert np.all(codes[0, len(cases):] == 0)


def test_scale_range_and_edges(orc):
    x = np.zeros(32, dtype=np.float16)
    x[5] = -3.0  # amax 3 = 1.5 * 2^1: X = -1 (byte 126), -3 / 0.5 = -6
    codes, e8 = orc.quantize_rows_mx8(x[None])
    assert e8[0, 0] == 126 and codes[0, 5] == 15
    # the smallest fp16 subnormal: X = -26 (no clamp), 2^-24 / 2^-26 = 4 -> index 6
    x = np.zeros(32, dtype=np.float16)
    x[0] = np.float16(2.0 ** -24)
    codes, e8 = orc.quantize_rows_mx8(x[None])
    assert e8[0, 0] == 101 and codes[0, 0] == 6
    # the largest fp16: 65504 = 1.999 * 2^15, X = 13 (byte 140), 7.996 saturates to 6
    x[0] = np.float16(65504.0)
    codes, e8 = orc.quantize_rows_mx8(x[None])
    assert e8[0, 0] == 140 and codes[0, 0] == 7
    # all zero: byte 127, codes 0
    codes, e8 = orc.quantize_rows_mx8(np.zeros((1, 32), np.float16))
    assert e8[0, 0] == 127 and np.all(codes == 0)


def test_brute_force_nearest(orc):
    rng = np.random.default_rng(31)
    for trial in range(60):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 3)).astype(np.float16)
        if trial % 7 == 0:
            x[rng.integers(0, 128, 5)] *= 20
        if trial % 11 == 0:
            x[:32] = 0.0
        codes, e8 = orc.quantize_rows_mx8(x[None])
        xf = x.astype(np.float64)
        for p in range(4):
            seg = xf[32 * p:32 * (p + 1)]
            amax = np.abs(seg).max()
            if amax == 0:
                assert e8[0, p] == 127 and np.all(codes[0, 32 * p:32 * (p + 1)] == 0)
                continue
            s = 2.0 ** (int(e8[0, p]) - 127)
            assert 4.0 <= amax / s < 8.0
            for i in range(32):
                c = int(codes[0, 32 * p + i])
                a = abs(seg[i]) / s
                d = [abs(a - m) for m in E2M1]
                assert d[c & 7] == min(d), (a, c)
                if sum(1 for j in range(8) if d[j] == min(d)) > 1:
                    assert (c & 7) % 2 == 0
                assert (c & 8) == (8 if (seg[i] < 0 and (c & 7)) else 0)


def test_bit_positions_hand_worked(orc):
    # block of 16 tokens = 16 * 128 * 4 bits; chunk 16g + (t mod 16) of 128 bits
    assert orc.k_bitpos_mx8(0, 0, 128) == 0
    assert orc.k_bitpos_mx8(0, 1, 128) == 4
    assert orc.k_bitpos_mx8(1, 0, 128) == 128
    assert orc.k_bitpos_mx8(0, 32, 128) == 16 * 128
    assert orc.k_bitpos_mx8(15, 127, 128) == (16 * 3 + 15) * 128 + 31 * 4
    assert orc.k_bitpos_mx8(17, 33, 128) == 8192 + 17 * 128 + 4
    assert orc.k_bitpos_mx8(40, 70, 128) == 2 * 8192 + (16 * 2 + 8) * 128 + 6 * 4


def test_layout_is_the_fp4_mfma_operand(orc):
    """The 1 KB of a 16-token block, read as 64 lanes x 16 bytes, is the A
    operand of a 16x16x128 FP4 product: lane l holds row (token) l mod 16 and
    K = 32 * (l // 16) + j at nibble j (low nibble first); the E8M0 bytes are
    [token][block]."""
    w = Workload("mxq_layout", 1, 4, 1, 128, 48, 4, 4, 32, 4, 0, 41)
    inp = make_inputs(w)
    c = orc.Cache(orc.Shape(1, 4, 1, 128, 4, 4, 32, 64, kfmt=2))
    c.append(inp.K, inp.V, np.zeros(1, np.int32))
    codes, e8 = orc.quantize_rows_mx8(inp.K[0, 0])
    kc = c.k_codes
    for blk in range(3):
        lanes = kc[blk * 1024:(blk + 1) * 1024].reshape(64, 16)
        for l in range(64):
            r, g = l % 16, l // 16
            nib = np.stack([lanes[l] & 15, lanes[l] >> 4], axis=1).reshape(32)
            assert np.array_equal(nib, codes[16 * blk + r, 32 * g:32 * g + 32]), (blk, l)
    assert np.array_equal(c.k_scales_e8()[0, 0, :48], e8)
    assert np.all(kc[3 * 1024:] == 0) and np.all(c.k_scales_e8()[0, 0, 48:] == 0)
    # the bit address agrees with the operand reading
    for t, ch in [(0, 0), (5, 37), (47, 127), (16, 64)]:
        assert orc.get_bits(kc, orc.k_bitpos_mx8(t, ch, 128), 4) == codes[t, ch]


def _grid_rows(rng, shape):
    """fp16 rows whose every 32-block lies on the MX grid: E2M1 values times
    2^Y with one element at +-6 * 2^Y (so X = Y and quantisation is exact)."""
    vals = rng.choice(np.array(E2M1 + [-v for v in E2M1[1:]]), size=shape)
    nb = shape[-1] // 32
    Y = rng.integers(-6, 2, size=shape[:-1] + (nb,))
    v = vals.reshape(shape[:-1] + (nb, 32))
    v[..., 0] = np.where(rng.random(shape[:-1] + (nb,)) < 0.5, 6.0, -6.0)
    x = v * np.ldexp(1.0, Y)[..., None]
    return x.reshape(shape).astype(np.float16)


def test_grid_inputs_give_exact_scores(orc):
    """q and K on the MX grid: the FP4 scores are the plain dot products, so
    sigma and the k = 0 output follow from the fp16 inputs directly."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, L = 2, 8, 2, 70
    K = _grid_rows(rng, (B, Hkv, L, 128))
    q = _grid_rows(rng, (B, Hq, 128))
    V = rng.standard_normal((B, Hkv, L, 128)).astype(np.float16)
    c = orc.Cache(orc.Shape(B, Hq, Hkv, 128, 4, 4, 32, 96, kfmt=2))
    c.append(K, V, np.zeros(B, np.int32))
    vc, vs, vz = orc.quantize_rows(V, 32, 4)
    Vh = (np.repeat(vs.view(np.float16).astype(np.float64), 32, axis=-1) * vc
          + np.repeat(vz.view(np.float16).astype(np.float64), 32, axis=-1))
    r = c.decode(q, np.full(B, L), 0, want_approx=True)
    for b in range(B):
        for h in range(Hq):
            s = K[b, h // 4].astype(np.float64) @ q[b, h].astype(np.float64) / np.sqrt(128)
            p = np.exp(s - s.max())
            np.testing.assert_allclose(r["out_approx"][b, h], p @ Vh[b, h // 4] / p.sum(), rtol=1e-11, atol=1e-12)
        for kvh in range(Hkv):
            s = np.stack([K[b, kvh].astype(np.float64) @ q[b, h].astype(np.float64)
                          for h in range(4 * kvh, 4 * kvh + 4)]) / np.sqrt(128)
            # (the dot products are exact on both sides; only the 1/sqrt(D) product rounds)
            np.testing.assert_allclose(r["sigma"][b, kvh, :L], s.max(0), rtol=4e-16, atol=0)


@pytest.mark.parametrize("vb", [4, 2])
def test_fp4_query_scores_and_exact_correction(orc, vb):
    """Random inputs: sigma and the k = 0 output from numpy on the codes of
    both operands; the k = len output is plain fp16 attention (the exact
    logits keep the fp16 query); and the scores differ from those against the
    unquantised query (the query really is quantised)."""
    w = Workload("mxq", 2, 8, 2, 128, 150, 4, vb, 32, 10, 3, 43)
    inp = make_inputs(w)
    c = orc.Cache(orc.Shape(w.B, w.Hq, w.Hkv, 128, 4, vb, 32, 160, kfmt=2))
    c.append(inp.K, inp.V, np.zeros(w.B, np.int32))
    kc, ke = orc.quantize_rows_mx8(inp.K)
    Kh = _dequant(kc, ke)
    qc, qe = orc.quantize_rows_mx8(inp.q)
    qh = _dequant(qc, qe)
    vc, vs, vz = orc.quantize_rows(inp.V, 32, vb)
    Vh = (np.repeat(vs.view(np.float16).astype(np.float64), 32, axis=-1) * vc
          + np.repeat(vz.view(np.float16).astype(np.float64), 32, axis=-1))
    r = c.decode(inp.q, np.full(w.B, w.L), 0, want_approx=True, want_exact=True)
    q = inp.q.astype(np.float64)
    for b in range(w.B):
        for h in range(w.Hq):
            s = Kh[b, h // 4] @ qh[b, h] / np.sqrt(128)
            p = np.exp(s - s.max())
            np.testing.assert_allclose(r["out_approx"][b, h], p @ Vh[b, h // 4] / p.sum(), rtol=1e-11, atol=1e-12)
            se = inp.K[b, h // 4].astype(np.float64) @ q[b, h] / np.sqrt(128)
            pe = np.exp(se - se.max())
            np.testing.assert_allclose(r["out_exact"][b, h], pe @ inp.V[b, h // 4].astype(np.float64) / pe.sum(),
                                       rtol=1e-11, atol=1e-12)
        for kvh in range(w.Hkv):
            hs = range(4 * kvh, 4 * kvh + 4)
            s = np.stack([Kh[b, kvh] @ qh[b, h] for h in hs]).max(0) / np.sqrt(128)
            np.testing.assert_allclose(r["sigma"][b, kvh, :w.L], s, rtol=1e-12, atol=1e-12)
            s16 = np.stack([Kh[b, kvh] @ q[b, h] for h in hs]).max(0) / np.sqrt(128)
            assert np.abs(s16 - s).max() > 1e-3
    assert np.array_equal(c.k_scales_e8()[:, :, :w.L], ke)


def test_append_one_at_a_time_equals_bulk(orc):
    w = Workload("mxq_app", 2, 8, 2, 128, 40, 4, 2, 32, 4, 0, 44)
    inp = make_inputs(w)
    a = orc.Cache(orc.Shape(2, 8, 2, 128, 4, 2, 32, 64, kfmt=2))
    b = orc.Cache(orc.Shape(2, 8, 2, 128, 4, 2, 32, 64, kfmt=2))
    a.append(inp.K, inp.V, np.zeros(2, np.int32))
    for t in range(w.L):
        b.append(inp.K[:, :, t:t + 1], inp.V[:, :, t:t + 1], np.full(2, t, np.int32))
    for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
