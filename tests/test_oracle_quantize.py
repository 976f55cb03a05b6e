"""Pins for the oracle's 3-bit quantizer and the packed record layout.

Pages: "RotaryQuant ..." (arXiv 2608.08081), Abstract -- 3-bit scalar
quantization after the rotation, attention on packed 3-bit tensors.  The
quantizer's levels and the record layout are readings; they are pinned by
brute force, closed forms and hand-derived bytes.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_records():
    recs = {}
    with open(os.path.join(GOLDEN, "pack_records.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                name, hexs = line.split(":", 1)
                recs[name.strip()] = np.array([int(t, 16) for t in hexs.split()], dtype=np.uint8)
    return recs


def _identity_params():
    p = np.zeros((32, 8))
    p[:, 0] = 1.0
    p[:, 4] = 1.0
    return p


def _random_params(rng):
    g = rng.standard_normal((32, 2, 4))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    return g.reshape(32, 8)


def _brute_force_codes(xr):
    """Nearest of the 8 levels s*(k - 3.5), ties to the upper level."""
    a = np.max(np.abs(xr))
    s = a / 3.5
    if s == 0:
        return np.full(xr.shape, 4)
    levels = s * (np.arange(8) - 3.5)
    out = np.empty(xr.shape, dtype=np.int64)
    for i, v in enumerate(xr):
        dist = np.abs(v - levels)
        best = np.flatnonzero(dist == dist.min())
        out[i] = best.max()
    return out


def test_quantize_is_nearest_level_brute_force():
    rng = np.random.default_rng(10)
    for trial in range(30):
        p = _random_params(rng)
        x = rng.standard_normal(128) * rng.uniform(0.01, 100)
        codes, scales, xr, s = oracle.quantize(x, p)
        np.testing.assert_array_equal(codes, _brute_force_codes(xr))
        assert scales.dtype == np.float32 and scales == np.float32(np.max(np.abs(xr)) / 3.5)


def test_quantize_thresholds_go_up_and_extremes():
    # With the identity blocks, x' = H x, so x = H x' feeds chosen rotated values in directly.
    H = oracle.hadamard(128)
    xr = np.zeros(128)
    xr[0] = 3.5           # sets a = 3.5, s = 1
    xr[1] = -3.5
    xr[2] = 0.0           # threshold between codes 3 and 4 -> 4
    xr[3] = 1.0           # threshold between codes 4 and 5 -> 5
    xr[4] = -1.0          # threshold between codes 2 and 3 -> 3
    xr[5] = 0.999999      # just below -> 4
    xr[6] = 2.5           # level of code 6 exactly
    codes, scales, xr_got, s = oracle.quantize(H @ xr, _identity_params())
    assert s == pytest.approx(1.0, abs=1e-14)
    got = codes[:7].tolist()
    assert got[0] == 7 and got[1] == 0 and got[5] == 4 and got[6] == 6
    # thresholds land within rounding of fp64 H H = I; check the rule on the exact values
    for i, want in [(2, 4), (3, 5), (4, 3)]:
        u = xr_got[i] / s + 4
        assert abs(u - round(u)) < 1e-12
        assert codes[i] == min(7, max(0, int(np.floor(u))))
        assert codes[i] in (want - 1, want)


def test_quantize_scale_invariant_codes_and_zero_vector():
    rng = np.random.default_rng(11)
    p = _random_params(rng)
    x = rng.standard_normal((5, 128))
    c1, s1, _, _ = oracle.quantize(x, p)
    c2, s2, _, _ = oracle.quantize(x * 8.0, p)     # power of two: exact scaling
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_allclose(s2, s1 * 8.0, rtol=1e-7)
    cz, sz, _, _ = oracle.quantize(np.zeros(128), p)
    assert sz == 0.0 and np.all(cz == 4)


def test_quantize_error_bound():
    # Every rotated coordinate lies within s/2 of its level (mid-rise, uniform step s).
    rng = np.random.default_rng(12)
    p = _random_params(rng)
    x = rng.standard_t(3, size=(50, 128))
    codes, scales, xr, s = oracle.quantize(x, p)
    err = np.abs(xr - oracle.dequantize_rotated(codes, s))
    assert np.all(err <= s[:, None] / 2 * (1 + 1e-12))


@pytest.mark.parametrize("name", ["all7", "all0", "all4", "mod8", "c127is5", "c70is3", "c21is6", "c15is6",
                                  "c2is7", "c5is7"])
def test_pack_golden_records(name):
    recs = _golden_records()
    codes = np.zeros(128, dtype=np.uint8)
    if name == "all7":
        codes[:] = 7
    elif name == "all4":
        codes[:] = 4
    elif name == "mod8":
        codes[:] = np.arange(128) % 8
    elif name == "c127is5":
        codes[127] = 5
    elif name == "c70is3":
        codes[70] = 3
    elif name == "c21is6":
        codes[21] = 6
    elif name == "c15is6":
        codes[15] = 6
    elif name == "c2is7":
        codes[2] = 7
    elif name == "c5is7":
        codes[5] = 7
    np.testing.assert_array_equal(oracle.pack(codes), recs[name])
    np.testing.assert_array_equal(oracle.unpack(recs[name]), codes)


def test_pack_roundtrip_every_value_every_position():
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 8, size=(200, 128)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.unpack(oracle.pack(codes)), codes)
    for v in range(8):
        for pos in range(128):
            c = np.zeros(128, dtype=np.uint8)
            c[pos] = v
            r = oracle.pack(c)
            np.testing.assert_array_equal(oracle.unpack(r), c)
            assert int(np.unpackbits(r).sum()) == bin(v).count("1")   # bits conserved, none lost
    assert oracle.pack(codes).shape == (200, 48)
