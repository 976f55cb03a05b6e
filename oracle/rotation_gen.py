"""Seeded generator of rotation parameters (unit quaternion pairs), fp64 steps.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The HIP library's
``iq_make_rotation`` implements the same published generator independently;
this module is the check on it.

Source: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
Compressed-Space Attention" (arXiv 2608.08081), Abstract: 256 stored
parameters per head for the block-diagonal SO(4) rotation.  How those
parameters are drawn is not stated; reading: each block's left and right
quaternions are uniform on the 3-sphere.

Generator (a reading, chosen so two independent implementations agree bit
for bit using only IEEE +, -, *, / and sqrt):
  * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): the i-th 64-bit output
    (i = 0, 1, ...) is mix(seed + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64);
  * v = (z >> 11) * 2^-52 - 1, uniform on [-1, 1) (exact in fp64);
  * Marsaglia's method for a uniform point on S^3 (Ann. Math. Statist. 43,
    1972): draw (x1, x2) until s1 = x1^2 + x2^2 < 1, draw (x3, x4) until
    0 < s2 = x3^2 + x4^2 < 1, then f = sqrt((1 - s1) / s2) and the point is
    (x1, x2, x3 f, x4 f);
  * order: head, block, left quaternion then right quaternion; one running
    counter for the whole call; every component rounded to fp32 (nearest
    even).
"""
import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed, i):
    """i-th output of SplitMix64 started from ``seed`` (a counter-based form)."""
    z = (seed + (i + 1) * GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


class _Stream:
    def __init__(self, seed):
        self.seed = seed & MASK64
        self.i = 0

    def uniform_pm1(self):
        z = splitmix64(self.seed, self.i)
        self.i += 1
        return float(z >> 11) * 2.0 ** -52 - 1.0


def _point_on_s3(st):
    while True:
        x1 = st.uniform_pm1()
        x2 = st.uniform_pm1()
        s1 = x1 * x1 + x2 * x2
        if s1 < 1.0:
            break
    while True:
        x3 = st.uniform_pm1()
        x4 = st.uniform_pm1()
        s2 = x3 * x3 + x4 * x4
        if 0.0 < s2 < 1.0:
            break
    f = np.sqrt((1.0 - s1) / s2)
    return (x1, x2, x3 * float(f), x4 * float(f))


def make_rotation(seed, n_heads):
    """float32 [n_heads][32][8]: per block, q_L (4 values) then q_R (4 values)."""
    st = _Stream(seed)
    out = np.zeros((n_heads, 32, 8), dtype=np.float32)
    for h in range(n_heads):
        for b in range(32):
            out[h, b, 0:4] = np.array(_point_on_s3(st), dtype=np.float64).astype(np.float32)
            out[h, b, 4:8] = np.array(_point_on_s3(st), dtype=np.float64).astype(np.float32)
    return out
