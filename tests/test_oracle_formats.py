"""Pins of the quantizer variants (oracle/formats.py).

Hand-derived 2-bit and 4-bit records; the generic packing equals the pinned
3-bit packing; brute-force nearest levels for the uniform quantizers; the
Lloyd-Max table against a fresh Lloyd iteration and against Max's published
levels and errors (tests/golden/lloyd_max_gaussian.txt); the RMS scale; the
classic ordering of the quantization errors; and attention on "u3" equal to
the pinned decode attention.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _records():
    out = {}
    for line in open(os.path.join(GOLDEN, "pack_records_2_4.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            name, hexes = line.split(":")
            out[name] = np.array([int(h, 16) for h in hexes.split()], dtype=np.uint8)
    return out


def test_two_and_four_bit_records_match_hand_derived_bytes():
    rec = _records()
    i = np.arange(128)
    cases = {"b2_all3": (2, np.full(128, 3)), "b2_mod4": (2, i % 4),
             "b2_c127is2": (2, np.where(i == 127, 2, 0)), "b2_c9is1": (2, np.where(i == 9, 1, 0)),
             "b4_mod16": (4, i % 16), "b4_c5is9": (4, np.where(i == 5, 9, 0)),
             "b4_c126is15": (4, np.where(i == 126, 15, 0))}
    for name, (b, codes) in cases.items():
        np.testing.assert_array_equal(F.pack_bits(codes, b), rec[name], err_msg=name)
        np.testing.assert_array_equal(F.unpack_bits(rec[name], b), codes, err_msg=name)


def test_generic_packing_equals_the_three_bit_packing_and_round_trips():
    rng = np.random.default_rng(70)
    c3 = rng.integers(0, 8, size=(20, 128))
    np.testing.assert_array_equal(F.pack_bits(c3, 3), oracle.pack(c3))
    for b in (2, 3, 4):
        c = rng.integers(0, 2 ** b, size=(30, 128))
        r = F.pack_bits(c, b)
        assert r.shape == (30, 16 * b)
        np.testing.assert_array_equal(F.unpack_bits(r, b), c)


@pytest.mark.parametrize("fmt", ["u2", "u3", "u4"])
def test_uniform_formats_pick_the_nearest_level(fmt):
    b = F.bits(fmt)
    rng = np.random.default_rng(71 + b)
    y = rng.standard_normal((50, 128)) * np.exp(rng.uniform(-1, 1, size=(50, 1)))
    codes, scales, s, u = F.quantize_rotated(y, fmt)
    grid = np.arange(2 ** b) - (2 ** b - 1) / 2.0              # levels in units of s
    for r in range(50):
        lv = s[r] * grid
        d = np.abs(y[r][:, None] - lv[None, :])
        best = np.argmin(d + 1e-12 * np.arange(2 ** b)[None, ::-1], axis=1)   # ties go up
        np.testing.assert_array_equal(codes[r], best)
    # extremes: +-max|y| take the outermost codes; the scale is max|y| / (2^(b-1) - 1/2)
    a = np.max(np.abs(y), axis=1)
    np.testing.assert_allclose(s, a / (2 ** (b - 1) - 0.5), rtol=1e-15)
    am = np.argmax(np.abs(y), axis=1)
    top = codes[np.arange(50), am]
    assert np.all(top[y[np.arange(50), am] > 0] == 2 ** b - 1) and np.all(top[y[np.arange(50), am] < 0] == 0)
    z, zs, _, _ = F.quantize_rotated(np.zeros((1, 128)), fmt)
    assert zs[0] == 0 and np.all(z == 2 ** (b - 1))


def _golden_lloyd_max():
    rows = {}
    for line in open(os.path.join(GOLDEN, "lloyd_max_gaussian.txt")):
        if line.strip() and not line.startswith("#"):
            v = [float(t) for t in line.split()]
            rows[int(v[0])] = (v[1:-1], v[-1])
    return rows


def test_lloyd_max_levels_and_errors_match_max_and_a_fresh_lloyd_iteration():
    gold = _golden_lloyd_max()
    assert gold[2][0][0] == pytest.approx(math.sqrt(2 / math.pi), abs=1e-4)
    assert gold[2][1] == pytest.approx(1 - 2 / math.pi, abs=1e-4)
    for n, (pos, mse) in gold.items():
        L = F.lloyd_max_gaussian(n)
        np.testing.assert_allclose(L[n // 2:], pos, atol=6e-4)
        np.testing.assert_allclose(L[:n // 2], -np.array(pos[::-1]), atol=6e-4)
        assert F.gaussian_distortion(L) == pytest.approx(mse, abs=6e-5)
    # the format's table is Max's 8 levels as printed (3-4 significant decimals): equal to the
    # golden numbers, and within half a unit of the last printed digit of the fixed point
    np.testing.assert_array_equal(F.LLOYD_MAX_8[4:], gold[8][0])
    L8 = F.lloyd_max_gaussian(8)
    np.testing.assert_allclose(F.LLOYD_MAX_8, L8, atol=5e-4)
    assert F.gaussian_distortion(F.LLOYD_MAX_8) == pytest.approx(gold[8][1], abs=6e-5)


def test_lloyd_max_table_is_odd_so_four_bit_planes_span_it():
    # The decode builds each Lloyd-Max level from four exact operand planes of the code c
    # (c, c & 6, c & 4, parity(c)) plus a constant.  That spans a level table exactly when the
    # table is odd about the middle code (level 7 - c = -level c), as Max's is: the odd functions
    # of three bits are spanned by the bits and their parity.  Check the premise on the oracle's
    # table, and that the span holds it and fails for a table that is not odd.
    L = np.array(F.LLOYD_MAX_8)
    np.testing.assert_array_equal(L[::-1], -L)
    c = np.arange(8)
    basis = np.stack([c, c & 6, c & 4, (c ^ (c >> 1) ^ (c >> 2)) & 1, np.ones(8)], axis=1).astype(np.float64)
    coef, *_ = np.linalg.lstsq(basis, L, rcond=None)
    np.testing.assert_allclose(basis @ coef, L, atol=1e-12)
    bent = L.copy()
    bent[7] += 0.01
    coef_b, *_ = np.linalg.lstsq(basis, bent, rcond=None)
    assert np.max(np.abs(basis @ coef_b - bent)) > 1e-3


def test_lloyd_max_format_nearest_level_and_rms_scale():
    rng = np.random.default_rng(75)
    y = rng.standard_normal((40, 128)) * 3.0
    codes, scales, sigma, u = F.quantize_rotated(y, "lm3")
    np.testing.assert_allclose(sigma, np.sqrt(np.mean(y * y, axis=1)), rtol=1e-14)
    L = np.array(F.LLOYD_MAX_8)
    for r in range(40):
        d = np.abs(y[r][:, None] / sigma[r] - L[None, :])
        np.testing.assert_array_equal(codes[r], np.argmin(d + 1e-12 * np.arange(8)[None, ::-1], axis=1))
    ones = np.where(np.arange(128) % 2 == 0, 1.0, -1.0)[None]
    c1, s1, _, _ = F.quantize_rotated(ones * 2.0, "lm3")     # |y| = 2 everywhere: sigma = 2
    assert s1[0] == 2.0 and np.all(c1[0, ::2] == 5) and np.all(c1[0, 1::2] == 2)   # 1.0 is nearest 0.756 (code 5)
    z, zs, _, _ = F.quantize_rotated(np.zeros((1, 128)), "lm3")
    assert zs[0] == 0 and np.all(z == 4)
    np.testing.assert_allclose(F.levels(c1, s1, "lm3")[0, :2], [2 * 0.7560, -2 * 0.7560])


def test_error_ordering_on_gaussian_vectors():
    # more bits, less error; on Gaussian coordinates the Lloyd-Max codebook with the RMS scale
    # beats the uniform 3-bit absmax quantizer, and its error is close to Max's 0.03454
    y = np.random.default_rng(76).standard_normal((4000, 128))
    mse = {}
    for fmt in F.FORMATS:
        codes, scales, _, _ = F.quantize_rotated(y, fmt)
        mse[fmt] = np.mean((y - F.levels(codes, scales, fmt)) ** 2)
    assert mse["u2"] > mse["u3"] > mse["u4"]
    assert mse["lm3"] < mse["u3"]
    assert abs(mse["lm3"] - 0.03454) < 0.002


def test_u3_attention_is_the_pinned_decode_attention():
    rng = np.random.default_rng(77)
    p = rng.standard_normal((2, 2, 32, 2, 4))
    p = (p / np.linalg.norm(p, axis=-1, keepdims=True)).reshape(2, 2, 32, 8)
    k = rng.standard_normal((2, 2, 30, 128))
    v = rng.standard_normal((2, 2, 30, 128))
    q = rng.standard_normal((2, 4, 128))
    kc = np.zeros((2, 2, 30, 128), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((2, 2, 30), np.float32)
    vs = np.zeros_like(ks)
    for b in range(2):
        for g in range(2):
            kc[b, g], ks[b, g], _, _ = F.quantize_format(k[b, g], p[b, g], "u3")
            vc[b, g], vs[b, g], _, _ = F.quantize_format(v[b, g], p[b, g], "u3")
    lens = np.array([30, 17])
    np.testing.assert_allclose(F.decode_attention_format(q, kc, ks, vc, vs, p, lens, "u3"),
                               oracle.decode_attention(q, kc, ks, vc, vs, p, lens), rtol=1e-12, atol=1e-14)
    c_old, s_old, _, _ = oracle.quantize(k[0, 0], p[0, 0])
    np.testing.assert_array_equal(kc[0, 0], c_old)


def test_asymmetric_format_nearest_level_extremes_and_shift():
    rng = np.random.default_rng(78)
    y = rng.standard_normal((40, 128)) * np.exp(rng.uniform(-1, 1, size=(40, 1))) + rng.uniform(-3, 3, size=(40, 1))
    codes, sm, s, u = F.quantize_rotated(y, "a3")
    assert sm.shape == (40, 2) and F.scale_words("a3") == 2
    m, M = y.min(axis=1), y.max(axis=1)
    np.testing.assert_allclose(s, (M - m) / 7, rtol=1e-15)
    np.testing.assert_array_equal(sm[:, 1], m.astype(np.float32))
    # brute force: the nearest of the 8 levels m + s j, ties upward
    for r in range(40):
        lv = m[r] + s[r] * np.arange(8)
        d = np.abs(y[r][:, None] - lv[None, :])
        np.testing.assert_array_equal(codes[r], np.argmin(d + 1e-12 * np.arange(8)[None, ::-1], axis=1))
    # the minimum and maximum coordinates take codes 0 and 7 and are reconstructed exactly
    rows = np.arange(40)
    assert np.all(codes[rows, np.argmin(y, axis=1)] == 0) and np.all(codes[rows, np.argmax(y, axis=1)] == 7)
    x = F.levels(codes, np.stack([s, m], axis=-1), "a3")
    np.testing.assert_allclose(x[rows, np.argmin(y, axis=1)], m, rtol=0, atol=0)
    np.testing.assert_allclose(x[rows, np.argmax(y, axis=1)], M, rtol=1e-14)
    assert np.all(np.abs(y - x) <= s[:, None] / 2 * (1 + 1e-12))
    # a constant shift moves m and leaves the codes and the step unchanged (an absmax scale would not)
    c2, sm2, s2, _ = F.quantize_rotated(y + 10.0, "a3")
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_allclose(s2, s, rtol=1e-12)
    # hand-computed: the ramp 0..7 repeated is its own code with s = 1, m = 0; a constant vector
    # has s = 0, codes 0 and is reconstructed exactly
    ramp = (np.arange(128) % 8).astype(np.float64)
    c3, sm3, _, _ = F.quantize_rotated(ramp[None] * 0.5 - 1.0, "a3")
    np.testing.assert_array_equal(c3[0], np.arange(128) % 8)
    np.testing.assert_array_equal(sm3[0], np.float32([0.5, -1.0]))
    c4, sm4, _, _ = F.quantize_rotated(np.full((1, 128), -2.25), "a3")
    assert np.all(c4 == 0) and sm4[0, 0] == 0 and sm4[0, 1] == -2.25
    np.testing.assert_array_equal(F.levels(c4, sm4, "a3"), np.full((1, 128), -2.25))


def test_asymmetric_beats_symmetric_on_offset_data():
    # on zero-mean Gaussians the min/max range is at most twice the absmax, so the asymmetric step
    # is no larger; on data with an offset the symmetric absmax scale wastes its levels
    y = np.random.default_rng(79).standard_normal((2000, 128))
    for off, factor in ((0.0, 1.0), (3.0, 4.0)):
        mse = {}
        for fmt in ("u3", "a3"):
            codes, scales, _, _ = F.quantize_rotated(y + off, fmt)
            mse[fmt] = np.mean((y + off - F.levels(codes, scales, fmt)) ** 2)
        assert mse["a3"] * factor < mse["u3"], (off, mse)


def test_uniform_levels_hand_written_and_within_half_a_step():
    # the level of code c is s (c - (2^b - 1)/2): written out by hand for unit scale, so a
    # centre of 2^(b-1) instead of (2^b - 1)/2 fails here
    s = np.float32(1.0)
    hand = {"u2": [-1.5, -0.5, 0.5, 1.5],
            "u3": [-3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5],
            "u4": [-7.5, -6.5, -5.5, -4.5, -3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, 7.5]}
    for fmt, want in hand.items():
        n = len(want)
        codes = (np.arange(128) % n).astype(np.uint8)[None]
        got = F.levels(codes, np.array([s]), fmt)[0]
        np.testing.assert_array_equal(got, np.array(want * (128 // n)), err_msg=fmt)
    assert F.levels(np.full((1, 128), 15, np.uint8), np.array([2.0]), "u4")[0, 0] == 15.0
    assert F.levels(np.zeros((1, 128), np.uint8), np.array([2.0]), "u4")[0, 0] == -15.0
    assert F.levels(np.ones((1, 128), np.uint8), np.array([4.0]), "u2")[0, 0] == -2.0
    # every uniform format reconstructs each coordinate within half a step: |y - level(c)| <= s/2
    rng = np.random.default_rng(80)
    y = rng.standard_normal((60, 128)) * np.exp(rng.uniform(-2, 2, size=(60, 1)))
    for fmt in ("u2", "u3", "u4", "a3"):
        codes, scales, s_exact, _ = F.quantize_rotated(y, fmt)
        if fmt == "a3":
            sc = np.stack([s_exact, y.min(axis=1)], axis=-1)
        else:
            sc = s_exact
        err = np.abs(y - F.levels(codes, sc, fmt))
        assert np.all(err <= s_exact[:, None] / 2 * (1 + 1e-12)), fmt
    # Lloyd-Max: inside the outermost levels a coordinate is within half the gap to its neighbours
    codes, sig, sig_exact, u = F.quantize_rotated(y, "lm3")
    L = np.array(F.LLOYD_MAX_8)
    inner = (u > L[0]) & (u < L[-1])
    err = np.abs(u - L[codes])
    gap = np.diff(L).max() / 2
    assert np.all(err[inner] <= gap * (1 + 1e-12))
