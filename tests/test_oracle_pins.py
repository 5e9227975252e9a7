"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- hand-derived closed forms (tests/golden), an independent bit-level
reference built on Python big integers, exact rational arithmetic, a library
Hadamard matrix, and brute force on tiny inputs.  A dropped term, a wrong
sign, offset, bit order, group index or transposed operand in the oracle fails
at least one of them."""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle as O
import qg_synth as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent bit-level references (Python integers, no NumPy bit ops)
# ---------------------------------------------------------------------------
def bigint_unpack_group(words, bits):
    """Codes of one group from its 4*b words via one Python integer."""
    v = int.from_bytes(np.asarray(words, dtype="<u4").tobytes(), "little")
    return [(v >> (bits * j)) & ((1 << bits) - 1) for j in range(128)]


def bigint_trellis_tile(words16):
    """States of one 16x16 tile: the 768-bit stream as one integer, MSB first."""
    v = int.from_bytes(np.asarray(words16, dtype=">u2").tobytes(), "big")
    vv = (v << 768) | v                       # cyclic continuation
    out = []
    for i in range(256):
        start = 3 * i
        out.append((vv >> (1536 - start - 16)) & 0xFFFF)
    return out


def half_from_hex(h):
    return float(np.array([int(h, 16)], dtype=np.uint16).view(np.float16)[0])


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------
def test_unpack_golden_closed_forms():
    n_cases = 0
    with open(os.path.join(GOLD, "packing_closed_forms.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            b, words, codes = [p.strip() for p in line.split("|")]
            b = int(b)
            w = np.array([int(t, 16) for t in words.split()], dtype=np.uint32)
            assert w.size == 4 * b
            want = np.zeros(128, dtype=np.int64)
            for kv in codes.split():
                j, c = kv.split("=")
                want[int(j)] = int(c)
            got = O.unpack_uniform(w, 1, 128, b)[0]
            np.testing.assert_array_equal(got, want)
            n_cases += 1
    assert n_cases >= 9


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_unpack_matches_bigint_reference(bits):
    N, K = 5, 384
    w = S.uniform_code_words(N, K, bits, cfg_id=99, tensor_id=bits)
    codes = O.unpack_uniform(w, N, K, bits)
    G = K // 128
    ww = w.reshape(N, G, 4 * bits)
    for n in range(N):
        for g in range(G):
            ref = bigint_unpack_group(ww[n, g], bits)
            np.testing.assert_array_equal(codes[n, 128 * g:128 * g + 128], ref)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_unpack_round_trip(bits):
    rng = np.random.default_rng(5)
    # every value at every in-group position (3-bit hits all 8 word straddles)
    codes = np.array([[(j + v) % (1 << bits) for j in range(128)] for v in range(1 << bits)])
    np.testing.assert_array_equal(O.unpack_uniform(O.pack_uniform(codes, bits), codes.shape[0], 128, bits), codes)
    # random codes, several groups
    codes = rng.integers(0, 1 << bits, size=(7, 640))
    np.testing.assert_array_equal(O.unpack_uniform(O.pack_uniform(codes, bits), 7, 640, bits), codes)
    # words -> codes -> words (no padding: every word pattern is a valid group)
    w = rng.integers(0, 2**32, size=20 * 4 * bits, dtype=np.uint64).astype(np.uint32)
    np.testing.assert_array_equal(O.pack_uniform(O.unpack_uniform(w, 20, 128, bits), bits), w)


def test_three_bit_straddles_cover_all_word_boundaries():
    # fields that cross a 32-bit word boundary in a 3-bit group
    straddle = [j for j in range(128) if (3 * j) // 32 != (3 * j + 2) // 32]
    assert straddle == [10, 21, 42, 53, 74, 85, 106, 117]
    for j in straddle:
        codes = np.zeros((1, 128), dtype=np.int64)
        codes[0, j] = 5
        w = O.pack_uniform(codes, 3)
        assert bigint_unpack_group(w, 3)[j] == 5
        assert O.unpack_uniform(w, 1, 128, 3)[0, j] == 5


def test_mixed_rows_concatenate_in_order():
    K = 256
    cb = np.array([3, 4, 2, 3, 4], dtype=np.uint8)
    w = S.mixed_code_words(cb, K, cfg_id=98)
    off = O.row_word_offsets(cb, K)
    assert off[-1] == w.size
    got = O.unpack_mixed(w, cb, K)
    for n, b in enumerate(cb):
        seg = w[off[n]:off[n + 1]].reshape(2, 4 * int(b))
        ref = bigint_unpack_group(seg[0], int(b)) + bigint_unpack_group(seg[1], int(b))
        np.testing.assert_array_equal(got[n], ref)


# ---------------------------------------------------------------------------
# dequantisation
# ---------------------------------------------------------------------------
def test_dequant_golden_closed_forms():
    n = 0
    with open(os.path.join(GOLD, "dequant_closed_forms.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            b, c, sh, val = line.split()
            s = np.array([[int(sh, 16)]], dtype=np.uint16).view(np.float16)
            codes = np.full((1, 128), int(c))
            w = O.dequant_uniform(codes, s, int(b))
            assert w[0, 0] == float(val) and w[0, 127] == float(val)
            n += 1
    assert n >= 10


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequant_exact_for_every_fp16_scale(bits):
    """(c - o_b) * s against integer arithmetic: s = m * 2^(e-11) exactly, so
    w = (2c - (2^b - 1)) * m * 2^(e - 12) with an integer product.  Exhaustive over
    every finite positive fp16 scale and every code; also checks w fits fp32."""
    s16 = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)
    s = s16.astype(np.float64)
    f, e = np.frexp(s)                       # s = f * 2^e, f in [0.5, 1)
    m = (f * 2048).astype(np.int64)          # 11-bit integer significand
    assert np.all(np.ldexp(m.astype(np.float64), e - 11) == s)
    for c in range(1 << bits):
        codes = np.full((s.size, 128), c)
        w = O.dequant_uniform(codes, s.reshape(-1, 1), bits)[:, 0]
        exact = np.ldexp(((2 * c - ((1 << bits) - 1)) * m).astype(np.float64), e - 12)
        np.testing.assert_array_equal(w, exact)
        np.testing.assert_array_equal(w.astype(np.float32).astype(np.float64), w)


def test_dequant_group_index_and_rows():
    N, K, b = 3, 512, 3
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 8, size=(N, K))
    s = (rng.random((N, K // 128)) + 0.5).astype(np.float16)
    w = O.dequant_uniform(codes, s, b)
    for n in range(N):
        for k in range(0, K, 37):
            want = (Fraction(int(codes[n, k])) - Fraction(7, 2)) * Fraction(float(s[n, k // 128]))
            assert Fraction(w[n, k]) == want


@pytest.mark.parametrize("gs", [64, 32])
def test_small_scale_groups_reduce_to_group_128(gs):
    """Scales of 64 or 32 that repeat one value over each 128 give exactly the
    group-128 weights (the pinned case above)."""
    N, K, b = 4, 768, 3
    rng = np.random.default_rng(gs)
    codes = rng.integers(0, 8, size=(N, K))
    s128 = (rng.random((N, K // 128)) + 0.25).astype(np.float16)
    small = np.repeat(s128, 128 // gs, axis=1)
    assert small.shape == (N, K // gs)
    np.testing.assert_array_equal(O.dequant_uniform(codes, small, b), O.dequant_uniform(codes, s128, b))


@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("bits", [2, 4])
def test_small_scale_groups_one_scale_moves_one_span(gs, bits):
    """Doubling one scale of a row changes exactly that row's weights in one
    span of gs consecutive k, and doubles them (every c - o is non-zero)."""
    N, K = 3, 512
    codes = np.random.default_rng(7).integers(0, 1 << bits, size=(N, K))
    ones = np.ones((N, K // gs), dtype=np.float16)
    base = O.dequant_uniform(codes, ones, bits)
    for n0, i in ((0, 0), (2, K // gs - 1), (1, 5)):
        s = ones.copy()
        s[n0, i] = 2.0
        w = O.dequant_uniform(codes, s, bits)
        changed = np.argwhere(w != base)
        assert set(changed[:, 0]) == {n0}
        assert sorted(changed[:, 1]) == list(range(i * gs, (i + 1) * gs))
        np.testing.assert_array_equal(w[n0, i * gs:(i + 1) * gs], 2 * base[n0, i * gs:(i + 1) * gs])


@pytest.mark.parametrize("gs", [64, 32])
def test_small_scale_groups_brute_force(gs):
    """y with scale groups of 64 or 32 against exact rationals, summing span by
    span over the scale groups."""
    M, N, K, b = 2, 3, 256, 3
    x = S.activations(M, K, cfg_id=98, tensor_id=gs)
    s = S.scales(N, K, cfg_id=98, tensor_id=gs + 1, group=gs)
    w = S.uniform_code_words(N, K, b, cfg_id=98, tensor_id=gs + 2)
    y = O.gemv_uniform(x, w, s, N, K, b)
    ww = np.asarray(w).reshape(N, K // 128, 4 * b)
    o = Fraction(7, 2)
    for m in range(M):
        for n in range(N):
            cs = [c for g in range(K // 128) for c in bigint_unpack_group(ww[n, g], b)]
            acc = Fraction(0)
            for i in range(K // gs):
                sc = Fraction(float(s[n, i]))
                for k in range(i * gs, (i + 1) * gs):
                    acc += Fraction(float(x[m, k])) * (cs[k] - o) * sc
            assert abs(y[m, n] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc)))


# ---------------------------------------------------------------------------
# MXFP4 ("The Rock8", format table: E2M1 leaves, 2 exponent / 1 mantissa bit,
# UE8M0 scale 2^(e-127) per 32 elements, 17 bytes per block)
# ---------------------------------------------------------------------------
def test_e2m1_values():
    vals = [O.e2m1_value(c) for c in range(16)]
    # eight magnitudes: 0 and 1/2 (exponent 0), then 1, 1.5, 2, 3, 4, 6
    assert vals[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert vals[c | 8] == -vals[c]  # the sign bit only negates (-0 for code 8)
    assert math.copysign(1.0, vals[8]) == -1.0
    # a binary float: each exponent step doubles, each mantissa step adds half the
    # exponent's unit, the subnormal step equals the first normal's unit
    for e in (1, 2):
        assert vals[2 * e + 2] == 2 * vals[2 * e]
    assert vals[1] == vals[3] - vals[2]
    # 2 exponent bits and 1 mantissa bit leave 4 bits per element: 32 elements in
    # 16 bytes plus the scale byte = the format's 17-byte block
    assert 32 * 4 // 8 + 1 == 17


def test_e8m0_values():
    assert O.e8m0_value(127) == 1.0 and O.e8m0_value(128) == 2.0 and O.e8m0_value(126) == 0.5
    assert O.e8m0_value(0) == 2.0 ** -127 and O.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(O.e8m0_value(255))


def test_mxfp4_dequant_blocks_and_brute_force():
    """Each scale byte covers exactly 32 consecutive k of its row; products
    against exact rationals."""
    N, K, M = 3, 256, 2
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(N, K))
    e8 = rng.integers(120, 130, size=(N, K // 32)).astype(np.uint8)
    w = O.dequant_mxfp4(codes, e8)
    base = O.dequant_mxfp4(codes, np.full_like(e8, 127))
    for n0, i in ((0, 0), (2, 7), (1, 3)):
        e2 = np.full_like(e8, 127)
        e2[n0, i] = 128
        changed = np.argwhere(O.dequant_mxfp4(codes, e2) != base)
        nz = [k for k in range(i * 32, (i + 1) * 32) if codes[n0, k] & 7]
        assert sorted(changed[:, 1]) == nz and set(changed[:, 0]) <= {n0}
    words = O.pack_uniform(codes, 4)
    x = S.activations(M, K, cfg_id=99)
    y = O.gemv_mxfp4(x, words, e8, N, K)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(x[m, k])) * Fraction(O.e2m1_value(codes[n, k])) * Fraction(2) ** (int(e8[n, k // 32]) - 127)
            assert abs(y[m, n] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc)))
    assert np.all(w == base * np.repeat(2.0 ** (e8.astype(np.float64) - 127), 32, axis=1))


# ---------------------------------------------------------------------------
# MXFP6 ("The Rock8", format table: OCP E3M2 leaves, 3 exponent / 2 mantissa
# bits, four values per three bytes, UE8M0 scale 2^(e-127) per 32 elements,
# 25 bytes per block)
# ---------------------------------------------------------------------------
def test_e3m2_values():
    vals = [O.e3m2_value(c) for c in range(64)]
    # the 32 magnitudes of a 3-exponent-bit, 2-mantissa-bit float with bias 3:
    # exponent 0 subnormal in steps of 1/16, then each binade of four values
    mags = [Fraction(m, 16) for m in range(4)]
    for e in range(1, 8):
        mags += [Fraction(2) ** (e - 3) * (1 + Fraction(m, 4)) for m in range(4)]
    assert [Fraction(v) for v in vals[:32]] == mags
    assert vals[31] == 28.0 and vals[1] == 0.0625 and vals[4] == 0.25  # largest, smallest subnormal, smallest normal
    for c in range(32):
        assert vals[c | 32] == -vals[c]  # bit 5 only negates (-0 for code 32)
    assert math.copysign(1.0, vals[32]) == -1.0
    # binary-float structure: each exponent step doubles, the subnormal step
    # equals the first normal binade's step, values increase with the code
    for c in range(4, 28):
        assert vals[c + 4] == 2 * vals[c]
    assert vals[1] == vals[5] - vals[4]
    assert all(vals[c] < vals[c + 1] for c in range(31))
    # 6 bits per element: 32 elements in 24 bytes plus the scale byte = the
    # format's 25-byte block
    assert 32 * 6 // 8 + 1 == 25


def test_mxfp6_stream_four_values_per_three_bytes():
    """Elements 4i..4i+3 of the 6-bit stream fill bytes 3i..3i+2 (LSB first),
    checked against a Python-integer reference; pack/unpack are inverses."""
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 64, size=(3, 256))
    words = O.pack_uniform(codes, 6)
    assert words.size == 3 * 2 * 24
    raw = np.asarray(words, dtype="<u4").tobytes()
    for n in range(3):
        for i in range(64):  # byte triple i of row n
            v = int.from_bytes(raw[n * 192 + 3 * i: n * 192 + 3 * i + 3], "little")
            assert [(v >> (6 * j)) & 63 for j in range(4)] == list(codes[n, 4 * i: 4 * i + 4])
    for n in range(3):
        for g in range(2):
            assert bigint_unpack_group(words[(n * 2 + g) * 24:(n * 2 + g + 1) * 24], 6) == list(codes[n, 128 * g: 128 * g + 128])
    assert np.array_equal(O.unpack_uniform(words, 3, 256, 6), codes)


def test_mxfp6_dequant_blocks_and_brute_force():
    """Each scale byte covers exactly 32 consecutive k of its row; products
    against exact rationals."""
    N, K, M = 3, 256, 2
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 64, size=(N, K))
    e8 = rng.integers(118, 132, size=(N, K // 32)).astype(np.uint8)
    w = O.dequant_mxfp6(codes, e8)
    base = O.dequant_mxfp6(codes, np.full_like(e8, 127))
    for n0, i in ((0, 0), (2, 7), (1, 3)):
        e2 = np.full_like(e8, 127)
        e2[n0, i] = 126
        changed = np.argwhere(O.dequant_mxfp6(codes, e2) != base)
        nz = [k for k in range(i * 32, (i + 1) * 32) if codes[n0, k] & 31]
        assert sorted(changed[:, 1]) == nz and set(changed[:, 0]) <= {n0}
    words = O.pack_uniform(codes, 6)
    x = S.activations(M, K, cfg_id=98)
    y = O.gemv_mxfp6(x, words, e8, N, K)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(x[m, k])) * Fraction(O.e3m2_value(codes[n, k])) * Fraction(2) ** (int(e8[n, k // 32]) - 127)
            assert abs(y[m, n] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc)))
    assert np.all(w == base * np.repeat(2.0 ** (e8.astype(np.float64) - 127), 32, axis=1))
    # a NaN scale byte makes exactly its block NaN
    e3 = e8.copy()
    e3[1, 2] = 255
    nan = np.isnan(O.dequant_mxfp6(codes, e3))
    assert nan[1, 64:96].all() and nan.sum() == 32


# ---------------------------------------------------------------------------
# contraction: brute force with exact rationals
# ---------------------------------------------------------------------------
def brute_gemv(x16, words, s16, N, K, bits):
    xs = [[Fraction(float(v)) for v in row] for row in x16]
    G = K // 128
    ww = np.asarray(words).reshape(N, G, 4 * bits)
    o = Fraction((1 << bits) - 1, 2)
    out = []
    for xr in xs:
        row = []
        for n in range(N):
            acc = Fraction(0)
            for g in range(G):
                sc = Fraction(float(s16[n, g]))
                cs = bigint_unpack_group(ww[n, g], bits)
                for j in range(128):
                    acc += xr[128 * g + j] * (cs[j] - o) * sc
            row.append(acc)
        out.append(row)
    return out


@pytest.mark.parametrize("bits,K,N,M", [(3, 128, 4, 1), (3, 256, 3, 2), (2, 384, 2, 1), (4, 256, 2, 2)])
def test_gemv_brute_force_exact(bits, K, N, M):
    x = S.activations(M, K, cfg_id=97, tensor_id=bits)
    s = S.scales(N, K, cfg_id=97, tensor_id=10 + bits)
    w = S.uniform_code_words(N, K, bits, cfg_id=97, tensor_id=20 + bits)
    y = O.gemv_uniform(x, w, s, N, K, bits)
    ref = brute_gemv(x, w, s, N, K, bits)
    for m in range(M):
        for n in range(N):
            r = float(ref[m][n])
            assert abs(y[m, n] - r) <= 1e-13 * max(1.0, abs(r))


def test_gemv_closed_forms():
    K, N, b = 512, 8, 3
    G = K // 128
    x = S.activations(2, K, cfg_id=96)
    s = S.scales(N, K, cfg_id=96)
    xs = x.astype(np.float64).reshape(2, G, 128).sum(-1)          # [M][G]
    for c in (0, 5, 7):
        codes = np.full((N, K), c)
        y = O.gemv_uniform(x, O.pack_uniform(codes, b), s, N, K, b)
        want = (c - 3.5) * (xs @ s.astype(np.float64).T)
        np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
    # one-hot x picks a weight column: y[n] = w[n][k]
    codes = np.random.default_rng(2).integers(0, 8, size=(N, K))
    w = O.pack_uniform(codes, b)
    for k in (0, 127, 128, 300, 511):
        e = np.zeros((1, K), dtype=np.float16)
        e[0, k] = 1.0
        y = O.gemv_uniform(e, w, s, N, K, b)[0]
        np.testing.assert_array_equal(y, (codes[:, k] - 3.5) * s[:, k // 128].astype(np.float64))
    # x = 0 gives exactly 0
    assert np.all(O.gemv_uniform(np.zeros((1, K), np.float16), w, s, N, K, b) == 0.0)


def test_gemv_rows_subset_matches_full():
    N, K, b = 64, 384, 3
    x = S.activations(3, K, cfg_id=95)
    s = S.scales(N, K, cfg_id=95)
    w = S.uniform_code_words(N, K, b, cfg_id=95)
    full = O.gemv_uniform(x, w, s, N, K, b)
    rows = np.array([0, 5, 17, 63])
    np.testing.assert_array_equal(O.gemv_uniform_rows(x, w, s, N, K, b, rows), full[:, rows])


def test_gemv_mixed_matches_uniform_rows():
    K = 256
    cb = S.column_bits(40, 0.2, 4, cfg_id=94)
    assert int((cb == 4).sum()) == 8
    x = S.activations(2, K, cfg_id=94)
    s = S.scales(40, K, cfg_id=94)
    w = S.mixed_code_words(cb, K, cfg_id=94)
    y = O.gemv_mixed(x, w, s, cb, K)
    off = O.row_word_offsets(cb, K)
    for n in range(40):
        b = int(cb[n])
        yn = O.gemv_uniform(x, w[off[n]:off[n + 1]], s[n:n + 1], 1, K, b)
        np.testing.assert_array_equal(y[:, n:n + 1], yn)


# ---------------------------------------------------------------------------
# Hadamard rotation
# ---------------------------------------------------------------------------
def test_hadamard_matches_scipy_sylvester():
    H = O.hadamard128()
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(128) * 2.0 ** -3.5)


def test_rotation_closed_forms_and_involution():
    vals = {}
    with open(os.path.join(GOLD, "hadamard_closed_forms.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    e0 = np.zeros((1, 256))
    e0[0, 128] = 1.0                                   # e_0 of the second group
    r = O.rotate(e0)
    assert np.all(r[0, :128] == 0.0)
    np.testing.assert_allclose(r[0, 128:], vals["e0_entry"], rtol=0, atol=1e-16)
    ones = np.ones((1, 128))
    r = O.rotate(ones)[0]
    assert abs(r[0] - vals["ones_entry0"]) < 1e-12 and np.all(np.abs(r[1:]) < 1e-12)
    # involution H(Hx) = x (2^-3.5 is irrational, so up to fp64 rounding)
    x = S.activations(3, 384, cfg_id=93).astype(np.float64)
    np.testing.assert_allclose(O.rotate(O.rotate(x)), x, rtol=0, atol=4e-15 * np.abs(x).max())


def test_rotation_uses_per_group_blocks():
    x = S.activations(1, 256, cfg_id=92).astype(np.float64)
    H = scipy.linalg.hadamard(128) / math.sqrt(128)
    want = np.concatenate([H @ x[0, :128], H @ x[0, 128:]])
    np.testing.assert_allclose(O.rotate(x)[0], want, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# trellis
# ---------------------------------------------------------------------------
def _golden_trellis_tiles():
    cases = []
    with open(os.path.join(GOLD, "trellis_closed_forms.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, pat, states = [p.strip() for p in line.split("|")]
            w = np.zeros(48, dtype=np.uint16)
            if pat.startswith("all "):
                w[:] = int(pat.split()[1], 16)
            elif pat.startswith("repeat "):
                p = [int(t, 16) for t in pat.split()[1:]]
                w[:] = np.array(p * (48 // len(p)), dtype=np.uint16)
            else:
                first = pat.split()[0]
                idx, val = first.split("=")
                w[int(idx.replace("word", ""))] = int(val, 16)
            want = {int(a): int(b, 16) for a, b in (kv.split("=") for kv in states.split())}
            cases.append((name, w, want))
    return cases


def test_trellis_golden_closed_forms():
    cases = _golden_trellis_tiles()
    assert len(cases) == 5
    for name, w, want in cases:
        st = O.trellis_states(w.reshape(1, 1, 48), 16, 16)        # [n=r][k=c]
        for i, v in want.items():
            r, c = divmod(i, 16)
            assert int(st[r, c]) == v, (name, i)
        ref = bigint_trellis_tile(w)
        for i, v in want.items():
            assert ref[i] == v, (name, i)


def test_trellis_matches_bigint_and_recurrence():
    N, K = 32, 48
    words = S.trellis_words(N, K, cfg_id=91)
    st = O.trellis_states(words, N, K)
    for tn in range(N // 16):
        for tk in range(K // 16):
            ref = bigint_trellis_tile(words[tn, tk])
            v = int.from_bytes(words[tn, tk].astype(">u2").tobytes(), "big")
            for i in range(256):
                r, c = divmod(i, 16)
                assert int(st[16 * tn + r, 16 * tk + c]) == ref[i]
                # shift-register recurrence, including the wrap 255 -> 0
                nxt = ref[(i + 1) % 256]
                pos = (3 * i + 16) % 768
                three = 0
                for u in range(3):
                    three = (three << 1) | ((v >> (767 - ((pos + u) % 768))) & 1)
                assert nxt == ((ref[i] << 3) | three) & 0xFFFF


def test_trellis_dequant_uses_codebook_and_group_scale():
    N, K = 16, 256
    words = S.trellis_words(N, K, cfg_id=90)
    cb = S.codebook(cfg_id=90)
    s = S.scales(N, K, cfg_id=90)
    st = O.trellis_states(words, N, K)
    w = O.trellis_dequant(st, cb, s)
    for n in (0, 7, 15):
        for k in (0, 127, 128, 255):
            assert w[n, k] == float(cb[st[n, k]]) * float(s[n, k // 128])
            assert w[n, k] == float(np.float32(cb[st[n, k]]) * np.float32(s[n, k // 128]))


def test_trellis_gemv_brute_force():
    N, K = 16, 128
    words = S.trellis_words(N, K, cfg_id=89)
    cb = S.codebook(cfg_id=89)
    s = S.scales(N, K, cfg_id=89)
    x = S.activations(1, K, cfg_id=89)
    y = O.gemv_trellis(x, words, cb, s, N, K)
    H = scipy.linalg.hadamard(128) / math.sqrt(128)
    xr = H @ x[0].astype(np.float64)
    for n in range(N):
        acc = []
        for k in range(K):
            tk, c = divmod(k, 16)
            r = n % 16
            state = bigint_trellis_tile(words[n // 16, tk])[16 * r + c]
            acc.append(xr[k] * float(cb[state]) * float(s[n, 0]))
        assert abs(y[0, n] - math.fsum(acc)) <= 1e-12 * max(1.0, abs(y[0, n]))


# ---------------------------------------------------------------------------
# MLP
# ---------------------------------------------------------------------------
def test_mlp_brute_force_tiny():
    H, I = 128, 256
    rng = np.random.default_rng(3)
    wg = rng.standard_normal((I, H)) * 0.05
    wu = rng.standard_normal((I, H)) * 0.05
    wd = rng.standard_normal((H, I)) * 0.05
    x = S.activations(1, H, cfg_id=88)
    out = O.mlp(x, wg, wu, wd)[0]
    xv = x[0].astype(np.float64)
    h = []
    for i in range(I):
        g = math.fsum(xv * wg[i])
        u = math.fsum(xv * wu[i])
        h.append(g / (1.0 + math.exp(-g)) * u)
    for n in range(H):
        ref = math.fsum(np.array(h) * wd[n])
        assert abs(out[n] - ref) <= 1e-12 * max(1.0, abs(ref))
    assert np.all(O.mlp(np.zeros((1, H)), wg, wu, wd) == 0.0)


def test_silu_identities():
    """SiLU(z) = z * sigmoid(z), pinned by identities that do not retype it:
    the tanh form z (1 + tanh(z / 2)) / 2, the odd part SiLU(z) - SiLU(-z) = z,
    slope 1/2 at 0, the asymptotes, and the stationary point z* (where the
    derivative vanishes, which forces SiLU(z*) = z* + 1)."""
    z = np.linspace(-30.0, 30.0, 1201)
    # (1 + tanh) cancels for large negative z: compare absolutely there
    np.testing.assert_allclose(O.silu(z), z * (1.0 + np.tanh(z / 2.0)) / 2.0, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert O.silu(np.array([0.0]))[0] == 0.0
    h = 1e-7
    assert abs(O.silu(np.array([h]))[0] / h - 0.5) < 1e-7
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-15
    assert 0.0 > O.silu(np.array([-40.0]))[0] > -1e-15
    from scipy.optimize import minimize_scalar
    r = minimize_scalar(lambda t: float(O.silu(np.array([t]))[0]), bracket=(-3.0, -1.0, 0.0), tol=1e-12)
    assert abs(float(O.silu(np.array([r.x]))[0]) - (r.x + 1.0)) < 1e-10
    assert -1.2785 < r.x < -1.2784


# ---------------------------------------------------------------------------
# mixed-precision mask (20 % of columns) and its bits/weight
# ---------------------------------------------------------------------------
def test_mixed_mask_counts_and_bpw():
    gu = S.column_bits(17408, 0.2, 4, cfg_id=S.CFG_MLP, tensor_id=S.T_MASK)
    dn = S.column_bits(5120, 0.2, 2, cfg_id=S.CFG_MLP, tensor_id=S.T_MASK + 100)
    assert int((gu == 4).sum()) == 3482 and int((gu == 3).sum()) == 17408 - 3482
    assert int((dn == 2).sum()) == 1024 and int((dn == 3).sum()) == 4096
    K_gu, K_dn = 5120, 17408
    bytes_gu = (int(gu.astype(np.int64).sum()) * K_gu) // 8 + 17408 * (K_gu // 128) * 2
    bytes_dn = (int(dn.astype(np.int64).sum()) * K_dn) // 8 + 5120 * (K_dn // 128) * 2
    assert bytes_gu == 37044480 and bytes_dn == 32587776
    total = 2 * bytes_gu + bytes_dn
    assert total == 106676736
    bpw = total * 8 / (2 * 17408 * 5120 + 5120 * 17408)
    assert abs(bpw - 3.1917) < 5e-5


def test_normwise_error_metric():
    r = np.array([[1.0, -4.0, 2.0]])
    y = np.array([[1.0, -4.002, 2.001]])
    assert abs(O.normwise_rel_err(y, r) - 0.002 / 4.0) < 1e-15


def test_trellis_row_subset_is_a_restriction():
    """The spot-check helper equals the full trellis product on the chosen rows."""
    N, K = 64, 256
    w = S.trellis_words(N, K, cfg_id=3)
    cb = S.codebook(cfg_id=3)
    sc = S.scales(N, K, cfg_id=3)
    x = S.activations(2, K, cfg_id=3)
    full = O.gemv_trellis(x, w, cb, sc, N, K)
    rows = np.array([0, 5, 17, 40, 63])
    np.testing.assert_allclose(O.gemv_trellis_rows(x, w, cb, sc, N, K, rows), full[:, rows], rtol=1e-12, atol=1e-12)
