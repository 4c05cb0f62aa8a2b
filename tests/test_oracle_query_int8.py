"""Pins of the oracle's INT8-query scores (O1q; HACK review on Pith, Eq. (4)).

HACK takes both operands of Q.K^T in quantised form and forms the product on
the integer codes plus correction terms.  Here the query partition is
symmetric (q ~= s*q', q' in [-127, 127], zero point 0), so for a key partition
x_hat = s_k*k' + z_k Eq. (4) keeps two terms:
    q_hat . x_hat = s*s_k*(q' . k') + s*z_k*sum(q').
Pinned by: brute force (q' is the nearest grid point), the quantisation error
bound, the extreme element, a query already on the grid (the scores then equal
the pinned fp16-query scores exactly), and Eq. (4) evaluated in exact rational
arithmetic from the oracle's own codes.
"""
from fractions import Fraction

import numpy as np
import pytest

from bit_kv_attention_amd.synth import Workload, make_inputs


def _workload(**kw):
    base = dict(name="t", B=1, Hq=4, Hkv=1, D=128, L=70, kbits=4, vbits=4, group=32,
                k=8, planted=0, seed=5)
    base.update(kw)
    return Workload(**base)


@pytest.mark.parametrize("g", [32, 64])
def test_codes_are_nearest_grid_points(orc, g):
    rng = np.random.default_rng(3)
    for trial in range(40):
        scale = 10.0 ** rng.uniform(-4, 2)
        q = (rng.standard_normal(128) * scale).astype(np.float16)
        if trial == 0:
            q[:] = 0  # all-zero partitions: scale 0, codes 0
        codes, scales = orc.quantize_query(q, g)
        qf = q.astype(np.float64)
        for p in range(128 // g):
            seg = qf[p * g:(p + 1) * g]
            amax = np.abs(seg).max()
            s = float(scales[p])
            assert s == float(np.float32(amax) / np.float32(127))
            cp = codes[p * g:(p + 1) * g].astype(np.int64)
            if amax == 0:
                assert np.all(cp == 0)
                continue
            # the extreme element lands on +-127
            i = int(np.argmax(np.abs(seg)))
            assert cp[i] == (127 if seg[i] > 0 else -127)
            # brute force over every code: q' minimises |s*n - q| (ties within
            # one fp32 rounding may go either way)
            grid = s * np.arange(-127, 128, dtype=np.float64)
            for c in range(g):
                err = np.abs(grid - seg[c])
                best = err.min()
                assert err[cp[c] + 127] <= best + 2 * abs(seg[c]) * 2.0 ** -24 + 1e-300
                assert abs(s * cp[c] - seg[c]) <= 0.5 * s * (1 + 2.0 ** -20)


def test_query_on_the_grid_gives_the_fp16_query_scores(orc):
    """q = n / 64 with integer |n| <= 127 and 127 in every partition: the scale
    is exactly 1/64, the codes are n, and the INT8-query scores, selection and
    outputs equal the fp16-query ones bit for bit."""
    w = _workload()
    inp = make_inputs(w)
    rng = np.random.default_rng(9)
    n = rng.integers(-127, 128, size=(w.B, w.Hq, w.D))
    n[..., ::32] = 127
    inp.q = (n / 64.0).astype(np.float16)
    cap = 96
    c = orc.Cache(orc.Shape(w.B, w.Hq, w.Hkv, w.D, w.kbits, w.vbits, w.group, cap))
    c.append(inp.K, inp.V, np.zeros(w.B, np.int32))
    codes, scales = orc.quantize_query(inp.q[0, 0], 32)
    assert np.all(scales == np.float32(1 / 64)) and np.array_equal(codes, n[0, 0])
    r0 = c.decode(inp.q, [w.L], w.k, want_approx=True)
    r8 = c.decode(inp.q, [w.L], w.k, want_approx=True, qbits=8)
    for key in ("sigma", "idx", "out", "out_approx"):
        assert np.array_equal(r0[key], r8[key], equal_nan=True), key


@pytest.mark.parametrize("kb,g", [(4, 32), (3, 32), (2, 64), (1, 64)])
def test_scores_follow_hack_eq4_exactly(orc, kb, g):
    """sigma from the oracle (G = 1, so sigma is the logit) against Eq. (4)
    with the query partition symmetric, evaluated in exact rationals from the
    key codes/meta and the query codes/scales."""
    w = _workload(Hq=1, kbits=kb, vbits=2, group=g, L=40)
    inp = make_inputs(w)
    cap = 64
    c = orc.Cache(orc.Shape(1, 1, 1, w.D, kb, 2, g, cap))
    c.append(inp.K, inp.V, np.zeros(1, np.int32))
    r = c.decode(inp.q, [w.L], 0, qbits=8)
    qc, qs = orc.quantize_query(inp.q[0, 0], g)
    kcodes, s16, z16 = orc.quantize_rows(inp.K[0, 0], g, kb)
    sk = s16.view(np.float16).astype(np.float64)
    zk = z16.view(np.float16).astype(np.float64)
    for t in range(w.L):
        tot = Fraction(0)
        for p in range(w.D // g):
            qp = [int(x) for x in qc[p * g:(p + 1) * g]]
            kp = [int(x) for x in kcodes[t, p * g:(p + 1) * g]]
            s, s_k, z_k = Fraction(float(qs[p])), Fraction(sk[t, p]), Fraction(zk[t, p])
            tot += s * s_k * sum(a * b for a, b in zip(qp, kp)) + s * z_k * sum(qp)
        ref = float(tot) / np.sqrt(w.D)
        assert abs(r["sigma"][0, 0, t] - ref) <= 1e-13 * (abs(ref) + 1e-3), t


def test_exact_logits_keep_the_fp16_query(orc):
    """Selecting every token makes the output exact attention with the fp16
    query whatever the approximate query is."""
    w = _workload(L=50)
    inp = make_inputs(w)
    c = orc.Cache(orc.Shape(w.B, w.Hq, w.Hkv, w.D, w.kbits, w.vbits, w.group, 64))
    c.append(inp.K, inp.V, np.zeros(w.B, np.int32))
    r0 = c.decode(inp.q, [w.L], w.L)
    r8 = c.decode(inp.q, [w.L], w.L, qbits=8)
    assert np.array_equal(r0["out"], r8["out"])
    # and with no selection the INT8 query moves the output only a little
    a0 = c.decode(inp.q, [w.L], 0)["out"]
    a8 = c.decode(inp.q, [w.L], 0, qbits=8)["out"]
    assert not np.array_equal(a0, a8)
    np.testing.assert_allclose(a8, a0, atol=0.05)
