"""Pins of the oracle's MXFP4 key codec (O1mx) and the scores built on it.

MXFP4 (Jet-QSparse abstract: FP4 keys; the block format of the OCP
Microscaling formats): 32 elements share a power-of-two scale 2^X with
X = floor(log2(amax)) - 2, and each element is an E2M1 number (magnitudes
0, 0.5, 1, 1.5, 2, 3, 4, 6).  Pinned by hand-derived blocks (ties to the even
mantissa, saturation, sign of zero), brute force over the E2M1 grid, the
scale's range, and attention over the dequantised keys computed in numpy
from the codes.
"""
import numpy as np
import pytest

from bit_kv_attention_amd.synth import Workload, make_inputs

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _val(code):
    return (-1.0 if code & 8 else 1.0) * E2M1[code & 7]


def test_e2m1_values(orc):
    for c in range(16):
        assert orc.e2m1_value(c) == _val(c)


def test_hand_derived_block(orc):
    """amax = 1.0 = 0.5 * 2^1, so X = 0 - 2 and the scale is 0.25; each entry
    is (x, x / 0.25, expected code)."""
    cases = [
        (1.0, 4.0, 6),        # exactly 4
        (-1.0, -4.0, 14),     # sign bit 8
        (0.3125, 1.25, 2),    # tie 1 | 1.5 -> even mantissa: 1
        (0.4375, 1.75, 4),    # tie 1.5 | 2 -> 2
        (0.0625, 0.25, 0),    # tie 0 | 0.5 -> 0
        (0.875, 3.5, 6),      # tie 3 | 4 -> 4
        (0.625, 2.5, 4),      # tie 2 | 3 -> 2
        (0.1875, 0.75, 2),    # tie 0.5 | 1 -> 1
        (0.7, 2.8, 5),        # nearest 3
        (-0.01, -0.04, 0),    # rounds to 0: no sign
        (0.125, 0.5, 1),      # exactly 0.5
        (-0.375, -1.5, 11),   # exactly -1.5
    ]
    x = np.zeros(32, dtype=np.float16)
    for i, (v, _, _) in enumerate(cases):
        x[i] = v
    codes, sc = orc.quantize_rows_mx(x[None], 32)
    assert float(sc.view(np.float16)[0, 0]) == 0.25
    for i, (v, r, want) in enumerate(cases):
        assert abs(float(np.float16(v)) / 0.25 - r) < 2e-3, v
        assert codes[0, i] == want, (v, codes[0, i], want)
    assert np.all(codes[0, len(cases):] == 0)


def test_saturation_and_scale_edges(orc):
    # amax = 1.9 = 0.95 * 2^1: X = -2, 1.9 / 0.25 = 7.6 clamps to 6
    x = np.zeros(32, dtype=np.float16)
    x[3] = 1.9
    x[4] = -1.5  # 6 exactly
    codes, sc = orc.quantize_rows_mx(x[None], 32)
    assert float(sc.view(np.float16)[0, 0]) == 0.25 and codes[0, 3] == 7 and codes[0, 4] == 15
    # all zero: scale 0, codes 0
    codes, sc = orc.quantize_rows_mx(np.zeros((1, 32), np.float16), 32)
    assert sc[0, 0] == 0 and np.all(codes == 0)
    # the smallest fp16 values: X clamped at -24 (2^-24 = the smallest subnormal)
    x = np.zeros(32, dtype=np.float16)
    x[0] = np.float16(2.0 ** -24)
    codes, sc = orc.quantize_rows_mx(x[None], 32)
    assert float(sc.view(np.float16)[0, 0]) == 2.0 ** -24 and codes[0, 0] == 2  # 1 * 2^-24


def test_brute_force_nearest(orc):
    rng = np.random.default_rng(21)
    for trial in range(60):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 2)).astype(np.float16)
        if trial % 7 == 0:
            x[rng.integers(0, 128, 5)] *= 20  # outliers in some blocks
        codes, sc = orc.quantize_rows_mx(x[None], 32)
        s = sc.view(np.float16)[0].astype(np.float64)
        xf = x.astype(np.float64)
        for p in range(4):
            seg = xf[32 * p:32 * (p + 1)]
            amax = np.abs(seg).max()
            if amax == 0:
                continue
            assert 4.0 <= amax / s[p] < 8.0  # X = floor(log2 amax) - 2
            for i in range(32):
                c = int(codes[0, 32 * p + i])
                a = abs(seg[i]) / s[p]
                d = [abs(a - m) for m in E2M1]
                assert d[c & 7] == min(d), (a, c)
                ties = [j for j in range(8) if d[j] == min(d)]
                if len(ties) > 1:
                    assert (c & 7) % 2 == 0
                assert (c & 8) == (8 if (seg[i] < 0 and (c & 7)) else 0)


@pytest.mark.parametrize("vb", [4, 2])
def test_attention_over_mx_keys(orc, vb):
    """k = 0: dense attention over the dequantised MXFP4 keys (numpy, from the
    codes) and affine values; k = len: exact attention, as for any codec."""
    w = Workload("mx", 2, 8, 2, 128, 150, 4, vb, 32, 10, 3, 33)
    inp = make_inputs(w)
    c = orc.Cache(orc.Shape(w.B, w.Hq, w.Hkv, 128, 4, vb, 32, 160, kfmt=1))
    c.append(inp.K, inp.V, np.zeros(w.B, np.int32))
    codes, sc = orc.quantize_rows_mx(inp.K, 32)
    vals = np.vectorize(_val)(codes.astype(np.int64))
    Kh = vals * np.repeat(sc.view(np.float16).astype(np.float64), 32, axis=-1)
    vc, vs, vz = orc.quantize_rows(inp.V, 32, vb)
    Vh = (np.repeat(vs.view(np.float16).astype(np.float64), 32, axis=-1) * vc
          + np.repeat(vz.view(np.float16).astype(np.float64), 32, axis=-1))
    r = c.decode(inp.q, np.full(w.B, w.L), 0, want_exact=True)
    q = inp.q.astype(np.float64)
    for b in range(w.B):
        for h in range(w.Hq):
            s = Kh[b, h // 4] @ q[b, h] / np.sqrt(128)
            p = np.exp(s - s.max())
            np.testing.assert_allclose(r["out"][b, h], p @ Vh[b, h // 4] / p.sum(), rtol=1e-11, atol=1e-12)
        for kvh in range(w.Hkv):
            sh = np.stack([Kh[b, kvh] @ q[b, h] / np.sqrt(128) for h in range(4 * kvh, 4 * kvh + 4)])
            np.testing.assert_allclose(r["sigma"][b, kvh, :w.L], sh.max(0), rtol=1e-12, atol=1e-12)
    # codes in the cache are the codec's, at the K4 bit positions
    for t in (0, 77, 149):
        for ch in (0, 31, 64, 127):
            got = orc.get_bits(c.k_codes, orc.k_bitpos(t, ch, 128, 4), 4)
            assert got == codes[0, 0, t, ch]
