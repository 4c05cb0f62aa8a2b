"""Pins of the oracle's storage layout (O2) and append (O1+O2).

The layout is this library's own convention (the pages give none); the pins
check it against hand-worked positions, closed forms built independently in
Python, and the partition property (every bit of a tile belongs to exactly one
(token, channel)).
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_bit_positions(orc):
    with open(os.path.join(GOLD, "layout_examples.json")) as f:
        ex = json.load(f)
    for e in ex["k"]:
        assert orc.k_bitpos(e["t"], e["c"], 128, e["bits"]) == e["bitpos"], e
    for e in ex["v"]:
        assert orc.v_bitpos(e["t"], e["c"], 128, e["bits"]) == e["bitpos"], e


@pytest.mark.parametrize("bits", [2, 4])
def test_v_tile_is_a_partition(orc, bits):
    D = 128
    owner = np.full(32 * D * bits, -1, dtype=np.int64)
    for r in range(32):
        for c in range(D):
            p = orc.v_bitpos(r, c, D, bits)
            assert np.all(owner[p:p + bits] == -1)
            owner[p:p + bits] = r * D + c
    assert np.all(owner >= 0)
    # the next tile starts right after
    assert orc.v_bitpos(32, 0, D, bits) == 32 * D * bits


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_k_block_is_a_partition(orc, bits):
    D = 128
    owner = np.full(16 * D * bits, -1, dtype=np.int64)
    for r in range(16):
        for c in range(D):
            p = orc.k_bitpos(r, c, D, bits)
            assert np.all(owner[p:p + bits] == -1)
            owner[p:p + bits] = r * D + c
    assert np.all(owner >= 0)
    assert orc.k_bitpos(16, 0, D, bits) == 16 * D * bits


def k_block_closed_form(codes16, bits):
    """The bytes of one 16-token K block built as one little-endian integer:
    chunk (e, r) at chunk index 16*e + r holds, for g = 0..3, the field
    sum_j code[r][32g + 8e + j] << (bits*j) at bit offset 8*bits*g."""
    fb = 8 * bits
    val = 0
    for e in range(4):
        for r in range(16):
            chunk = 0
            for g in range(4):
                field = 0
                for j in range(8):
                    field |= int(codes16[r, 32 * g + 8 * e + j]) << (bits * j)
                chunk |= field << (fb * g)
            val |= chunk << (4 * fb * (16 * e + r))
    nbytes = 16 * 128 * bits // 8
    return np.frombuffer(val.to_bytes(nbytes, "little"), dtype=np.uint8)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_k_blocks_closed_form(orc, bits):
    """Packed K blocks equal an independently built integer (see
    k_block_closed_form); the last block is partly filled and the rows past
    the appended tokens stay zero."""
    rng = np.random.default_rng(bits)
    s = orc.Shape(B=1, Hq=1, Hkv=1, D=128, kbits=bits, vbits=2, group=32, cap=64)
    cache = orc.Cache(s)
    n = 40
    K = rng.standard_normal((1, 1, n, 128)).astype(np.float16)
    V = rng.standard_normal((1, 1, n, 128)).astype(np.float16)
    cache.append(K, V, [0])
    codes, _, _ = orc.quantize_rows(K[0, 0], 32, bits)
    full = np.zeros((48, 128), dtype=np.int64)
    full[:n] = codes
    bb = 16 * 128 * bits // 8
    for blk in range(3):
        want = k_block_closed_form(full[16 * blk:16 * blk + 16], bits)
        assert np.array_equal(cache.k_codes[blk * bb:(blk + 1) * bb], want), blk
    if bits == 4:  # nibble form of chunk (e=0, r=0): bytes 4g+i = channels 32g+2i, 32g+2i+1
        chunk = cache.k_codes[:16]
        want = np.array([codes[0, 32 * g + 2 * i] | (codes[0, 32 * g + 2 * i + 1] << 4)
                         for g in range(4) for i in range(4)], dtype=np.uint8)
        assert np.array_equal(chunk, want)
    assert not cache.k_codes[3 * bb:].any()


@pytest.mark.parametrize("bits,group", [(2, 32), (4, 32), (2, 64), (4, 64)])
def test_v_roundtrip_and_meta_and_shadow(orc, bits, group):
    rng = np.random.default_rng(20 + bits)
    s = orc.Shape(B=2, Hq=4, Hkv=2, D=128, kbits=4, vbits=bits, group=group, cap=96)
    cache = orc.Cache(s)
    n = 70
    K = rng.standard_normal((2, 2, n, 128)).astype(np.float16)
    V = rng.standard_normal((2, 2, n, 128)).astype(np.float16)
    cache.append(K, V, [0, 0])
    ub = 96 * 128 * bits // 8
    for u in range(4):
        b, h = divmod(u, 2)
        codes, vs, vz = orc.quantize_rows(V[b, h], group, bits)
        base = cache.v_codes[u * ub:(u + 1) * ub]
        for t in range(0, n, 7):
            for c in range(0, 128, 5):
                assert orc.get_bits(base, orc.v_bitpos(t, c, 128, bits), bits) == codes[t, c]
        mp = cache.v_meta_planes()[b, h]  # [grp][cap]
        assert np.array_equal(mp[:, :n].T & 0xFFFF, vs)
        assert np.array_equal(mp[:, :n].T >> 16, vz)
        assert not mp[:, n:].any()
        sh = cache.v_shadow.reshape(2, 2, 96, 128)[b, h]
        assert np.array_equal(sh[:n], V[b, h].view(np.uint16))
        ksh = cache.k_shadow.reshape(2, 2, 96, 128)[b, h]
        assert np.array_equal(ksh[:n], K[b, h].view(np.uint16))


def test_append_one_at_a_time_equals_bulk(orc):
    """Groups are per token, so appending tokens one by one (with ragged
    per-sequence positions) gives the same bytes as one bulk append."""
    rng = np.random.default_rng(9)
    s = orc.Shape(B=2, Hq=2, Hkv=1, D=128, kbits=3, vbits=2, group=32, cap=64)
    n = 45
    K = rng.standard_normal((2, 1, n, 128)).astype(np.float16)
    V = rng.standard_normal((2, 1, n, 128)).astype(np.float16)
    bulk = orc.Cache(s)
    bulk.append(K, V, [0, 0])
    step = orc.Cache(s)
    step.append(K[:, :, :10], V[:, :, :10], [0, 0])
    for t in range(10, n):
        step.append(K[:, :, t:t + 1], V[:, :, t:t + 1], [t, t])
    for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_shadow", "v_shadow"):
        assert np.array_equal(getattr(bulk, name), getattr(step, name)), name
