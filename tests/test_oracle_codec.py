"""Pins of the oracle's codec (O1) and fp16 conversions, independent of the oracle itself.

The quantiser is the asymmetric per-group uniform one: zero point = group minimum,
step = range / (2^b - 1), x ~= s*x' + m (HACK review on Pith, Eq. (4) and
'What carries the argument'; TailorKV review on Pith, fp16 zero point and scale).
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _dequant64(codes, s16, z16, g):
    s = s16.view(np.float16).astype(np.float64)
    z = z16.view(np.float16).astype(np.float64)
    return np.repeat(s, g, axis=-1) * codes + np.repeat(z, g, axis=-1)


def test_f16_to_f32_all_patterns(orc):
    """Every fp16 bit pattern decodes like numpy's (independent) conversion."""
    L = orc.lib()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([L.orc_f16_to_f32(int(p)) for p in pats], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_rne_matches_numpy(orc):
    """Round-to-nearest-even fp32->fp16, including exact halfway cases, the
    subnormal range and overflow, against numpy's conversion."""
    L = orc.lib()
    rng = np.random.default_rng(5)
    vals = [rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000)]
    # exact midpoints between adjacent fp16 values (ties) across the range
    h = rng.integers(0, 0x7BFF, 4000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    vals.append(((lo + hi) / 2).astype(np.float32).astype(np.float64))
    vals.append(np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6,
                          2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25]))
    with np.errstate(over="ignore"):
        x = np.concatenate(vals).astype(np.float32)
    x = x[np.isfinite(x)]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([L.orc_f32_to_f16(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_golden_hand_examples(orc):
    """Hand-worked quantisation examples (tests/golden/codec_examples.json)."""
    with open(os.path.join(GOLD, "codec_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float16)[None, :]
        codes, s16, z16 = orc.quantize_rows(x, group=x.shape[1], bits=c["bits"])
        assert int(s16[0, 0]) == int(c["scale16"], 16), c["why"]
        assert int(z16[0, 0]) == int(c["zero16"], 16), c["why"]
        assert codes[0].tolist() == c["codes"], c["why"]


def test_one_element_group_is_exact(orc):
    """A 1-element group reproduces its value exactly."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 128)) * 3).astype(np.float16)
    x[0, :4] = [0.0, -0.0, 65504.0, 6e-8]
    for bits in (2, 3, 4):
        codes, s16, z16 = orc.quantize_rows(x, group=1, bits=bits)
        xh = _dequant64(codes, s16, z16, 1)
        assert np.array_equal(xh, x.astype(np.float64))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("g", [4, 32, 64, 128])
def test_error_within_half_step(orc, bits, g):
    """|x - x_hat| <= s16/2 per element, plus the fp32 rounding of (x - z)/s
    (at most 2^-22 of the larger magnitude)."""
    rng = np.random.default_rng(bits * 100 + g)
    x = (rng.standard_normal((200, 128)) * rng.choice([0.01, 1, 8, 300], (200, 1))).astype(np.float16)
    codes, s16, z16 = orc.quantize_rows(x, group=g, bits=bits)
    xh = _dequant64(codes, s16, z16, g)
    x64 = x.astype(np.float64)
    s = np.repeat(s16.view(np.float16).astype(np.float64), g, axis=-1)
    z = np.repeat(z16.view(np.float16).astype(np.float64), g, axis=-1)
    slack = 2.0 ** -22 * np.maximum(np.abs(x64), np.abs(z))
    err = np.abs(x64 - xh)
    # The half-step bound needs the stored scale to be an fp16 normal: a
    # subnormal scale carries too few bits, so (max-min)/s16 can exceed 2^b-1 by
    # more than half a code and the clamp costs more.  There the error is still
    # bounded by s16/2 + (2^b-1)*|s32 - s16| (fp32 scale before rounding).
    normal = s >= 2.0 ** -14
    assert np.all((err <= s / 2 + slack)[normal])
    xg = x64.reshape(x64.shape[0], -1, g)
    s32 = ((xg.max(-1) - xg.min(-1)).astype(np.float32) / np.float32((1 << bits) - 1)).astype(np.float64)
    s32 = np.repeat(s32, g, axis=-1)
    assert np.all(err <= s / 2 + ((1 << bits) - 1) * np.abs(s32 - s) + slack)
    assert codes.max() <= (1 << bits) - 1


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_min_and_max_hit_end_codes(orc, bits):
    """In every group with a nonzero scale the minimum codes to 0 and the
    maximum to 2^b - 1 ((max-min)/s16 = (2^b-1)(1 +- 2^-11))."""
    rng = np.random.default_rng(7 + bits)
    x = rng.standard_normal((300, 128)).astype(np.float16)
    g = 32
    codes, s16, _ = orc.quantize_rows(x, group=g, bits=bits)
    xg = x.reshape(300, 4, g)
    cg = codes.reshape(300, 4, g)
    for r in range(300):
        for j in range(4):
            if s16[r, j] == 0:
                continue
            assert cg[r, j, np.argmin(xg[r, j])] == 0
            assert cg[r, j, np.argmax(xg[r, j])] == (1 << bits) - 1


def test_power_of_two_scaling_is_equivariant(orc):
    """Scaling a row by 2^j (staying normal in fp16) scales s and z by 2^j
    and leaves the codes unchanged."""
    rng = np.random.default_rng(3)
    # magnitudes in [1/8, 4]: stays in the fp16 normal range after scaling by 2^-3..2^3
    x = (rng.choice([-1.0, 1.0], (100, 128)) * rng.uniform(0.125, 4, (100, 128))).astype(np.float16)
    c0, s0, z0 = orc.quantize_rows(x, 32, 3)
    for j in (-3, -1, 1, 3):
        xs = (x.astype(np.float64) * 2.0 ** j).astype(np.float16)
        assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) * 2.0 ** j)
        c1, s1, z1 = orc.quantize_rows(xs, 32, 3)
        assert np.array_equal(c1, c0)
        assert np.array_equal(s1.view(np.float16).astype(np.float64), s0.view(np.float16).astype(np.float64) * 2.0 ** j)
        assert np.array_equal(z1.view(np.float16).astype(np.float64), z0.view(np.float16).astype(np.float64) * 2.0 ** j)


def test_planted_mistake_is_caught(orc):
    """The half-step bound would fail for a quantiser that truncated instead of
    rounding: check the bound is tight enough to notice (sanity of the pin)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 32)).astype(np.float16)
    codes, s16, z16 = orc.quantize_rows(x, 32, 4)
    s = s16.view(np.float16).astype(np.float64)
    z = z16.view(np.float16).astype(np.float64)
    trunc = np.clip(np.floor((x.astype(np.float64) - z) / s), 0, 15)
    err = np.abs(x.astype(np.float64) - (s * trunc + z))
    assert np.any(err > s / 2 + 1e-6)
