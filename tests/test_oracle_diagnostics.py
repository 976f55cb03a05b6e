"""Pins of the isotropy diagnostics oracle (oracle/diagnostics.py).

Kurtosis values with closed forms, a hand-worked quantization error, the
peak-to-average ratios of a spike before and after the WHT, transforms
checked against an independent butterfly and Hamilton products, a
permutation that shows which side the dense matrix acts on, and the
Gaussian value 3 on a large sample.
"""
import numpy as np
import pytest

from oracle import diagnostics as Dg
from oracle import make_rotation
from test_oracle_rotation import _fwht, _hamilton, _random_params


def _blocks_by_hamilton(x, params):
    """v -> q_L v conj(q_R) on every 4-coordinate block, by explicit Hamilton products."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for b in range(32):
        ql = params[b, 0:4] / np.linalg.norm(params[b, 0:4])
        qr = params[b, 4:8] / np.linalg.norm(params[b, 4:8])
        conj = qr * np.array([1.0, -1.0, -1.0, -1.0])
        for t in range(x.shape[0]):
            out[t, 4 * b:4 * b + 4] = _hamilton(_hamilton(ql, x[t, 4 * b:4 * b + 4]), conj)
    return out


def test_kurtosis_closed_forms():
    x = np.zeros((4, 128))
    x[:, 0] = [1.0, -1.0, 1.0, -1.0]            # two-point symmetric: kurtosis 1
    x[:, 1] = [5.0, 0.0, 0.0, 0.0]              # Bernoulli(1/4) scaled: (1 - 3pq) / pq = 7/3
    x[:, 2] = [-3.0, -1.0, 1.0, 3.0]            # m2 = 5, m4 = 41: 41/25
    x[:, 3] = 2.5                               # constant: variance 0, kurtosis reported as 0
    s = Dg.isotropy_stats(x, "none")
    assert s[0] == pytest.approx(1.0, abs=1e-12)
    assert s[1] == pytest.approx(7.0 / 3.0, abs=1e-12)
    assert s[2] == pytest.approx(41.0 / 25.0, abs=1e-12)
    assert s[3] == 0.0 and s[128 + 3] == 0.0
    assert s[128 + 2] == pytest.approx(5.0, abs=1e-12) and s[128 + 1] == pytest.approx(75.0 / 16.0, abs=1e-12)
    assert s[Dg.I_COUNT] == 4


def test_within_vector_kurtosis_and_papr_of_a_spike_before_and_after_the_wht():
    e0 = np.zeros((1, 128))
    e0[0, 0] = 2.0
    s = Dg.isotropy_stats(e0, "none")
    p = 1.0 / 128
    assert s[Dg.I_VEC_KURT] == pytest.approx((1 - 3 * p * (1 - p)) / (p * (1 - p)), rel=1e-12)   # 16003 / 127
    assert s[Dg.I_PAPR] == pytest.approx(128.0, rel=1e-12)
    w = Dg.isotropy_stats(e0, "wht")            # the spike becomes a constant vector
    assert w[Dg.I_PAPR] == pytest.approx(1.0, rel=1e-12)
    assert w[Dg.I_VEC_KURT] == 0.0
    assert w[Dg.I_REL_MSE] == pytest.approx(0.0, abs=1e-24)   # every entry is +-a: no error


def test_quantization_error_worked_example():
    # y = (3.5, 1, 0, ..., 0): s = 1; 3.5 -> code 7 (exact), 1 -> code 5 (level 1.5), 0 -> code 4
    # (level 0.5): error 0.25 + 126 * 0.25 = 31.75 over energy 13.25
    y = np.zeros((1, 128))
    y[0, 0], y[0, 1] = 3.5, 1.0
    s = Dg.isotropy_stats(y, "none")
    assert s[Dg.I_REL_MSE] == pytest.approx(31.75 / 13.25, rel=1e-12)
    assert Dg.isotropy_stats(np.zeros((3, 128)), "none")[Dg.I_REL_MSE] == 0.0
    assert np.all(Dg.isotropy_stats(np.zeros((0, 128)), "wht") == 0.0)


def test_transforms_against_independent_butterfly_and_hamilton_products():
    rng = np.random.default_rng(3)
    x = rng.standard_t(3, size=(64, 128))
    params = _random_params(rng)[0]
    h = _fwht(x)
    np.testing.assert_allclose(Dg.isotropy_stats(x, "wht"), Dg.isotropy_stats(h, "none"), rtol=1e-9, atol=1e-12)
    so4 = _blocks_by_hamilton(x, params)
    np.testing.assert_allclose(Dg.isotropy_stats(x, "so4", params), Dg.isotropy_stats(so4, "none"),
                               rtol=1e-9, atol=1e-12)
    both = _blocks_by_hamilton(h, params)        # WHT first, then the blocks
    np.testing.assert_allclose(Dg.isotropy_stats(x, "wht_so4", params), Dg.isotropy_stats(both, "none"),
                               rtol=1e-9, atol=1e-12)
    wrong_order = _fwht(_blocks_by_hamilton(x, params))
    assert not np.allclose(Dg.isotropy_stats(x, "wht_so4", params), Dg.isotropy_stats(wrong_order, "none"))


def test_dense_transform_acts_as_y_equals_t_x():
    # a permutation matrix P (P[i, perm[i]] = 1) gives y_i = x_perm[i]: per-coordinate statistics
    # are permuted by perm, not by its inverse
    rng = np.random.default_rng(4)
    x = rng.standard_normal((200, 128)) * np.exp(rng.uniform(-2, 2, size=128))
    perm = rng.permutation(128)
    P = np.zeros((128, 128))
    P[np.arange(128), perm] = 1.0
    sd, sn = Dg.isotropy_stats(x, "dense", dense=P), Dg.isotropy_stats(x, "none")
    np.testing.assert_allclose(sd[0:128], sn[0:128][perm], rtol=1e-12)
    np.testing.assert_allclose(sd[128:256], sn[128:256][perm], rtol=1e-12)
    assert not np.allclose(sd[128:256], sn[128:256][np.argsort(perm)])


def test_gaussian_kurtosis_is_three():
    x = np.random.default_rng(5).standard_normal((100000, 128))
    s = Dg.isotropy_stats(x, "none")
    assert np.all(np.abs(s[0:128] - 3.0) < 0.1)
    assert abs(np.mean(s[0:128]) - 3.0) < 0.01
    # the kurtosis of n = 128 Gaussian samples has mean close to 3 (n - 1) / (n + 1) = 3 - 6 / (n + 1)
    assert abs(s[Dg.I_VEC_KURT] - (3.0 - 6.0 / 129.0)) < 0.02


def test_rotation_isotropises_heavy_tails_and_outlier_channels():
    # The method's claim as a property: on Student-t(3) vectors and on vectors with a few large
    # channels the WHT + SO(4) rotation brings per-coordinate kurtosis towards 3 and cuts the
    # 3-bit quantization error.
    rng = np.random.default_rng(6)
    params = make_rotation(11, 1)[0]
    heavy = rng.standard_t(3, size=(4000, 128))
    chan = rng.standard_normal((4000, 128))
    chan[:, [5, 40, 77, 120]] *= 20.0
    for x in (heavy, chan):
        none, rot = Dg.isotropy_stats(x, "none"), Dg.isotropy_stats(x, "wht_so4", params)
        assert rot[Dg.I_REL_MSE] < 0.7 * none[Dg.I_REL_MSE]
        assert rot[Dg.I_PAPR] < none[Dg.I_PAPR]
    none, rot = Dg.isotropy_stats(heavy, "none"), Dg.isotropy_stats(heavy, "wht_so4", params)
    assert abs(np.mean(rot[0:128]) - 3.0) < abs(np.mean(none[0:128]) - 3.0)
