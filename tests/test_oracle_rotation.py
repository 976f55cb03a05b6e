"""Pins for the oracle's rotation: Walsh-Hadamard transform and SO(4) blocks.

The pages ("RotaryQuant ..." arXiv 2608.08081, Abstract) fix: a
Walsh-Hadamard transform *followed by* block-diagonal SO(4) rotations,
256 stored parameters per head against 16,384 for a dense rotation, and
O(d log d) work against O(d^2).  Everything else pinned here is textbook
mathematics.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_matrix(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


def _fwht(x):
    """Independent fast Walsh-Hadamard butterfly (in-place, natural order)."""
    x = np.array(x, dtype=np.float64)
    n = x.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x / np.sqrt(n)


def _hamilton(a, b):
    """Textbook Hamilton product of quaternions (w, x, y, z)."""
    a0, a1, a2, a3 = a
    b0, b1, b2, b3 = b
    return np.array([a0 * b0 - a1 * b1 - a2 * b2 - a3 * b3,
                     a0 * b1 + a1 * b0 + a2 * b3 - a3 * b2,
                     a0 * b2 - a1 * b3 + a2 * b0 + a3 * b1,
                     a0 * b3 + a1 * b2 - a2 * b1 + a3 * b0])


def _random_params(rng, n=1):
    g = rng.standard_normal((n, 32, 2, 4))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    return g.reshape(n, 32, 8)


def test_hadamard_h4_matches_sylvester_golden():
    H4 = oracle.hadamard(4) * 2.0
    np.testing.assert_array_equal(H4, _golden_matrix("hadamard4.txt"))


def test_hadamard_equals_fast_butterfly_and_is_orthogonal_involution():
    H = oracle.hadamard(128)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 128))
    np.testing.assert_allclose(x @ H.T, _fwht(x), atol=1e-13)
    np.testing.assert_allclose(H @ H.T, np.eye(128), atol=1e-13)
    np.testing.assert_array_equal(H, H.T)
    np.testing.assert_allclose(H @ np.eye(128)[0], np.full(128, 1 / np.sqrt(128)), atol=1e-15)


def test_hadamard_kronecker_factorisation():
    # H_128 = (I_32 (x) H_4)(H_32 (x) I_4): the two finest butterfly stages act inside
    # aligned blocks of 4, which is what lets a kernel fold them into the 4x4 blocks.
    lhs = oracle.hadamard(128)
    rhs = np.kron(np.eye(32), oracle.hadamard(4)) @ np.kron(oracle.hadamard(32), np.eye(4))
    np.testing.assert_allclose(lhs, rhs, atol=1e-14)


def test_block_is_left_times_conjugate_right_hamilton_product():
    rng = np.random.default_rng(1)
    for _ in range(20):
        ql, qr, v = rng.standard_normal((3, 4))
        ql /= np.linalg.norm(ql)
        qr /= np.linalg.norm(qr)
        ref = _hamilton(_hamilton(ql, v), oracle.quat_conj(qr))
        np.testing.assert_allclose(oracle.block_matrix(ql, qr) @ v, ref, atol=1e-14)


def test_block_is_so4_and_left_right_commute():
    rng = np.random.default_rng(2)
    for _ in range(20):
        a, b = rng.standard_normal((2, 4)) * 3.0   # not unit: block_matrix normalises
        M = oracle.block_matrix(a, b)
        np.testing.assert_allclose(M.T @ M, np.eye(4), atol=1e-13)
        assert abs(np.linalg.det(M) - 1.0) < 1e-12
        L = oracle.quat_left(a)
        Rm = oracle.quat_right(b)
        np.testing.assert_allclose(L @ Rm, Rm @ L, atol=1e-12)


def test_block_special_cases():
    one = np.array([1.0, 0, 0, 0])
    np.testing.assert_allclose(oracle.block_matrix(one, one), np.eye(4), atol=0)
    # q_L = q_R = q: fixes the real axis, rotates (x, y, z) like the textbook 3x3 matrix.
    q = np.array([np.sqrt(3) / 2, 0, 0, 0.5])
    M = oracle.block_matrix(q, q)
    np.testing.assert_allclose(M[0], one, atol=1e-15)
    np.testing.assert_allclose(M[:, 0], one, atol=1e-15)
    np.testing.assert_allclose(M[1:, 1:], _golden_matrix("quaternion_rotation.txt"), atol=1e-15)
    # q_L = (cos t, sin t, 0, 0), q_R = 1: left-isoclinic rotation by t in planes (0,1) and (2,3).
    t = 0.3
    M = oracle.block_matrix([np.cos(t), np.sin(t), 0, 0], one)
    c, s = np.cos(t), np.sin(t)
    ref = np.array([[c, -s, 0, 0], [s, c, 0, 0], [0, 0, c, -s], [0, 0, s, c]])
    np.testing.assert_allclose(M, ref, atol=1e-15)


def test_rotation_is_wht_then_blocks():
    # x = H e_i gives H x = e_i, so R x must be column i of blockdiag(M): this fails if the
    # composition order is swapped or the wrong block acts on the wrong coordinates.
    rng = np.random.default_rng(3)
    p = _random_params(rng)[0]
    H = oracle.hadamard(128)
    R = oracle.rotation_matrix(p)
    for i in [0, 5, 63, 64, 127]:
        col = R @ (H @ np.eye(128)[i])
        b = i // 4
        ref = np.zeros(128)
        ref[4 * b:4 * b + 4] = oracle.block_matrix(p[b, :4], p[b, 4:])[:, i % 4]
        np.testing.assert_allclose(col, ref, atol=1e-14)


def test_rotation_orthogonal_preserves_inner_products():
    rng = np.random.default_rng(4)
    p = _random_params(rng)[0].astype(np.float32)   # fp32-stored params, normalised inside
    R = oracle.rotation_matrix(p)
    np.testing.assert_allclose(R.T @ R, np.eye(128), atol=1e-12)
    q, k = rng.standard_normal((2, 128))
    assert abs(np.dot(R @ q, R @ k) - np.dot(q, k)) <= 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)
    assert abs(np.linalg.norm(R @ q) - np.linalg.norm(q)) <= 1e-12 * np.linalg.norm(q)


def test_parameter_and_operation_counts():
    # 256 stored parameters per head vs 16,384 for a dense rotation (pages, Abstract).
    p = np.zeros((32, 8))
    assert p.size == 256 and 128 * 128 == 16384
    # O(d log d): 7 butterfly stages of 128 add/sub plus 32 blocks of 16 multiply-adds,
    # against 16,384 multiply-adds for the dense product.
    fast_ops = int(np.log2(128)) * 128 + 32 * 16
    assert fast_ops == 1408 and fast_ops < 128 * 128 / 10


def test_rotate_uses_fp64_and_matches_dense_product():
    rng = np.random.default_rng(5)
    p = _random_params(rng)[0]
    x = rng.standard_normal((3, 128))
    R = oracle.rotation_matrix(p)
    np.testing.assert_allclose(oracle.rotate(x, p), x @ R.T, atol=1e-13)
    B = np.zeros((128, 128))
    for b in range(32):
        B[4 * b:4 * b + 4, 4 * b:4 * b + 4] = oracle.block_matrix(p[b, :4], p[b, 4:])
    np.testing.assert_allclose(oracle.rotate(x, p), (B @ _fwht(x).T).T, atol=1e-13)


@pytest.mark.parametrize("bits,val", [(0x3F80, 1.0), (0xC000, -2.0), (0x0000, 0.0), (0x7F7F, 3.3895313892515355e38),
                                      (0x0001, 9.183549615799121e-41)])
def test_bf16_conversion_exact(bits, val):
    assert oracle.bf16_bits_to_f64(np.array([bits]))[0] == val
