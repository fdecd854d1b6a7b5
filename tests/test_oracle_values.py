"""Pins of the oracle's value path (MSE-only value compression and decode
attention over packed keys and values) against what the mathematics fixes.

* codes are the nearest of the 2^b levels (brute force over all levels);
* the distortion over random unit vectors is Max's (1960) table MSE for
  2^b levels, and stays under e * 2^(-2b) [ICLR 2026 digest, Theorem 2];
* the packed value record holds b-bit codes and one half norm per value, the
  byte count of the community compression table [Qiita explainer, byte
  table], with bit positions checked by hand;
* decode attention: equal logits give the mean of the decoded values, a
  dominating logit gives that value, adding a constant to all logits changes
  nothing, zero values give zero.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_codes_are_nearest_level(bits):
    d = 64
    cb = O.make_codebook(d, bits, d, 3)
    lv, _ = O.value_quantizer(cb)
    rng = np.random.default_rng(bits)
    v = rng.standard_normal((300, d)) * np.exp(rng.normal(0, 0.5, d))
    e = O.encode_values(cb, v)
    nearest = np.argmin(np.abs(e.y[:, :, None] - lv[None, None, :]), axis=2)
    ok = ~e.code_flag
    assert np.array_equal(e.codes[ok], nearest[ok])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_distortion_matches_max_table(bits):
    ref = json.load(open(os.path.join(GOLDEN, "lloyd_max_gaussian.json")))[f"B{bits}"]["mse"]
    d = 128
    cb = O.make_codebook(d, bits, d, 9)
    x = _unit(np.random.default_rng(40 + bits), 6000, d)
    e = O.encode_values(cb, x)
    buf = O.pack_values(cb, e.codes[None], e.nu16[None])
    xhat = O.decode_values(cb, buf, 1, x.shape[0])[0] / e.nu16.astype(np.float64)[:, None]
    dist = np.mean(np.sum((x - xhat) ** 2, axis=1))
    assert abs(dist - ref) / ref < 0.03
    assert dist <= math.e * 2.0 ** (-2 * bits)


def test_value_record_layout_by_hand():
    """d = 64, 3 bits (groups of 2 values, 6 bits), N = 2: one tile of 16
    values, 64 slots of 48 bits = 96 words, then the two half norms.
    Coordinate 33 sits in slot 34 (32 * 1 + 16 * 0 + 2 // 2 = 33) and
    coordinate 0 in slot 0.  Code 5 of value 1 at coordinate 33: value 1 is
    i = 1 of group 0, planes 0 and 2 = bits 2 * 0 + 1 and 2 * 2 + 1 of slot
    34, stream bits 48 * 34 + 1 = 1633 and 1637 = bits 1 and 5 of word 51.
    Code 2 of value 0 at coordinate 0: plane 1 = bit 2 of slot 0 = bit 2 of
    word 0."""
    d, bits = 64, 3
    cb = O.make_codebook(d, bits, d, 1)
    assert O.value_group_size(bits) == 2 and O.value_group_size(4) == 2
    assert O.value_slot_coordinate(34) == 33 and O.value_slot_coordinate(0) == 0
    assert sorted(O.value_slot_coordinate(np.arange(d)).tolist()) == list(range(d))
    codes = np.zeros((1, 2, d), np.uint8)
    codes[0, 1, 33] = 5
    codes[0, 0, 0] = 2
    nu16 = np.array([[1.5, -0.0]], np.float16)
    buf = O.pack_values(cb, codes, nu16)
    assert buf.size == O.value_packed_nbytes(cb, 1, 2) == 96 * 4 + 2 * 2
    w = buf[: 96 * 4].view(np.uint32)
    expect = np.zeros(96, np.uint32)
    expect[51] = (1 << 1) | (1 << 5)
    expect[0] = 1 << 2
    assert np.array_equal(w, expect)
    assert buf[-4:].view(np.uint16).tolist() == [0x3E00, 0x8000]
    c2, n2 = O.unpack_values(cb, buf, 1, 2)
    assert np.array_equal(c2, codes) and np.array_equal(n2.view(np.uint16), nu16.view(np.uint16))


def test_value_record_layout_four_bits_by_hand():
    """4 bits: groups of 2 values (8 bits).  Code 9 (0b1001) of value 3 at
    coordinate 17 (slot 3: 32 * 0 + 16 * 1 + 2 // 2): value 3 is i = 1 of
    group 1, planes 0 and 3 = bits 8 + 2 * 0 + 1 and 8 + 2 * 3 + 1 of the
    64-bit slot 3, stream bits 201 and 207 = bits 9 and 15 of word 6."""
    d, bits = 32, 4
    cb = O.make_codebook(d, bits, d, 1)
    codes = np.zeros((1, 5, d), np.uint8)
    codes[0, 3, 17] = 9
    buf = O.pack_values(cb, codes, np.zeros((1, 5), np.float16))
    assert buf.size == 16 * 4 * 32 // 8 + 2 * 5
    w = buf[: 16 * 4 * 32 // 8].view(np.uint32)
    expect = np.zeros(64, np.uint32)
    expect[6] = (1 << 9) | (1 << 15)
    assert np.array_equal(w, expect)


def test_value_records_round_trip_ragged():
    """Random codes for N = 1, 15, 16, 17, 40 values: unpack(pack) is the
    identity, and the words equal those of the tiles padded with code-0
    values."""
    rng = np.random.default_rng(8)
    for bits in (2, 3, 4):
        cb = O.make_codebook(128, bits, 128, 3)
        for N in (1, 15, 16, 17, 40):
            codes = rng.integers(0, 1 << bits, size=(2, N, 128), dtype=np.uint8)
            nu16 = rng.standard_normal((2, N)).astype(np.float16)
            buf = O.pack_values(cb, codes, nu16)
            c2, n2 = O.unpack_values(cb, buf, 2, N)
            assert np.array_equal(c2, codes) and np.array_equal(n2.view(np.uint16), nu16.view(np.uint16))
            NP = ((N + 15) // 16) * 16
            padded = np.zeros((2, NP, 128), np.uint8)
            padded[:, :N] = codes
            full = O.pack_values(cb, padded, np.zeros((2, NP), np.float16))
            nw = buf.size - 2 * 2 * N
            assert nw == full.size - 2 * 2 * NP and np.array_equal(buf[:nw], full[:nw])


def test_value_bytes_reproduce_the_compression_table():
    """Qwen2.5-3B shape (36 layers x 2 KV heads x 8192 tokens, d = 128): key +
    value records over the fp16 K+V size give 3.82 / 5.02 / 7.31 x at 4 / 3 /
    2 bits (the community table prints 3.8 / 5.0 / 7.3 x)."""
    n = 36 * 2 * 8192
    fp16 = 2 * n * 128 * 2
    for bits, ratio in ((4, 3.8), (3, 5.0), (2, 7.3)):
        cb = O.make_codebook(128, bits, 128, 42)
        kv = O.packed_nbytes(cb, 1, n) + O.value_packed_nbytes(cb, 1, n)
        assert round(fp16 / kv, 1) == ratio


def _vbuf(cb, rng, G, N):
    v = rng.standard_normal((G * N, cb.d)) * 3.0
    e = O.encode_values(cb, v)
    return O.pack_values(cb, e.codes.reshape(G, N, cb.d), e.nu16.reshape(G, N))


def test_attention_special_cases():
    d = 64
    cb = O.make_codebook(d, 3, d, 2)
    rng = np.random.default_rng(5)
    G, N, Qg = 2, 9, 3
    vb = _vbuf(cb, rng, G, N)
    vh = O.decode_values(cb, vb, G, N)
    # equal logits: the mean of the decoded values
    out = O.attention_from_logits(cb, np.full((G, Qg, N), 0.7), vb, G, N)
    assert np.allclose(out, np.broadcast_to(vh.mean(axis=1)[:, None, :], out.shape), atol=1e-12)
    # one logit 2000 above the rest (scaled by 1/8 at d = 64): that value
    lg = rng.standard_normal((G, Qg, N))
    lg[:, :, 4] += 2000.0
    out = O.attention_from_logits(cb, lg, vb, G, N)
    assert np.allclose(out, np.broadcast_to(vh[:, 4][:, None, :], out.shape), atol=1e-9)
    # shift invariance, and the scale argument
    lg = rng.standard_normal((G, Qg, N)) * 5
    a = O.attention_from_logits(cb, lg, vb, G, N, scale=0.3)
    b = O.attention_from_logits(cb, lg + 123.0, vb, G, N, scale=0.3)
    assert np.allclose(a, b, atol=1e-12)
    # convex combination: every output lies inside the values' coordinate range
    assert np.all(a <= vh.max(axis=1)[:, None, :] + 1e-12) and np.all(a >= vh.min(axis=1)[:, None, :] - 1e-12)
    # zero values give zero
    zb = O.pack_values(cb, np.zeros((G, N, d), np.uint8), np.zeros((G, N), np.float16))
    assert np.all(O.attention_from_logits(cb, lg, zb, G, N) == 0.0)


def test_zero_value_rule():
    cb = O.make_codebook(32, 2, 32, 1)
    v = np.zeros((2, 32))
    v[1, 3] = 1e-12
    e = O.encode_values(cb, v)
    assert not e.codes.any() and np.all(e.nu16 == 0) and e.zero.all()
