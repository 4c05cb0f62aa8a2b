"""Shared helpers of the GPU parity tests: run the same step on both sides and
apply the acceptance rules.

Acceptance (the build's contract):
  * packed codes, scales, zeros and shadow rows: bit-exact;
  * top-k sets: equal size; any token in one set but not the other must have
    an oracle score within 1e-4 (relative) of the oracle's k-th score (plus a
    1e-6 absolute floor for scores near zero);
  * outputs: |gpu - ref| <= 2e-3 or <= 1e-2 * |ref| elementwise, checked
    against the oracle on the GPU's own selected set (arithmetic) and on the
    oracle's selected set (end to end).
"""
from __future__ import annotations

import numpy as np

import oracle
from bit_kv_attention_amd import binding as bk
from bit_kv_attention_amd.step import DecodeStep
from bit_kv_attention_amd.synth import Workload, make_inputs, make_new_tokens

ATOL, RTOL = 2e-3, 1e-2


def assert_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    ok = (err <= ATOL) | (err <= RTOL * np.abs(ref))
    if not ok.all():
        i = np.unravel_index(np.argmax(np.where(ok, 0, err)), err.shape)
        raise AssertionError(f"{what}: {int((~ok).sum())} elements out of tolerance; worst at {i}: "
                             f"gpu={got[i]!r} ref={ref[i]!r}")
    return float(err.max()) if err.size else 0.0


def assert_topk_near_tie(gpu_idx, orc_idx, sigma_orc, n, what=""):
    g = set(int(x) for x in gpu_idx if x >= 0)
    o = set(int(x) for x in orc_idx if x >= 0)
    assert len(g) == len(o), f"{what}: set sizes {len(g)} vs {len(o)}"
    if g == o:
        return 0
    kk = len(o)
    sk = np.sort(sigma_orc[:n])[::-1][kk - 1]
    bound = 1e-4 * abs(sk) + 1e-6
    for t in g ^ o:
        assert 0 <= t < n, f"{what}: index {t} outside [0, {n})"
        assert abs(sigma_orc[t] - sk) <= bound, f"{what}: token {t} sigma {sigma_orc[t]} vs k-th {sk}"
    return len(g ^ o)


def torch_dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dev())


def build_pair(w: Workload, L: int, cap: int | None = None, tweak=None):
    """Both caches holding the same L-1 prefill tokens, plus the step's new
    token, q and the layout.  tweak(inp), if given, may change the seeded
    inputs in place before they are packed.  Returns dict."""
    cap = cap or ((L + 31) // 32) * 32
    inp = make_inputs(w, L=L - 1) if L > 1 else None
    if tweak is not None and inp is not None:
        tweak(inp)
    k1, v1 = make_new_tokens(w, 1, inp.outlier_ch if inp else make_inputs(w, L=1).outlier_ch)
    lay = bk.make_layout(w.B, w.Hq, w.Hkv, cap, w.kbits, w.vbits, group=w.group, query_bits=w.query_bits,
                         key_format=w.key_format)
    gc = bk.allocate_cache(lay)
    oc = oracle.Cache(oracle.Shape(w.B, w.Hq, w.Hkv, 128, w.kbits, w.vbits, w.group, cap, w.key_format))
    q = inp.q if inp else make_inputs(w, L=1).q
    if L > 1:
        bk.kv_pack_append(lay, gc, to_dev(inp.K), to_dev(inp.V), L - 1, [0] * w.B)
        oc.append(inp.K, inp.V, np.zeros(w.B, np.int32))
    return dict(w=w, L=L, cap=cap, lay=lay, gc=gc, oc=oc, q=q, k1=k1[0], v1=v1[0], inp=inp)


def gpu_buffers(gc):
    return {n: getattr(gc, n).cpu().numpy().view(np.uint8) for n in
            ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow")}


def orc_buffers(oc):
    return {n: getattr(oc, n).view(np.uint8) for n in
            ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow")}


def run_step(P, lens, k):
    """Append the new token at lens[b]-1 on both sides, then run the GPU
    attention over lens[b] tokens.  Returns the GPU results as numpy."""
    import torch
    w = P["w"]
    pos = [max(int(x) - 1, 0) for x in lens]
    bk.kv_pack_append(P["lay"], P["gc"], to_dev(P["k1"]), to_dev(P["v1"]), 1, pos)
    P["oc"].append(P["k1"], P["v1"], np.array(pos, np.int32))
    st = DecodeStep(P["lay"], k, int(max(lens)))
    out = st.attend(P["gc"], to_dev(P["q"]), lens)
    torch.cuda.synchronize()
    cap = P["cap"]
    return dict(out=out.cpu().numpy().reshape(w.B, w.Hq, 128),
                sigma=st.sigma.cpu().numpy().reshape(w.B, w.Hkv, cap),
                idx=st.idx.cpu().numpy().reshape(w.B, w.Hkv, max(k, 1))[:, :, :k])
