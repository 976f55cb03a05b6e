"""Isotropy diagnostics of the KV vectors under the rotation and its variants (fp64).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing on the product
path imports it, and it shares no code with the HIP path.

Source: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
Compressed-Space Attention" (arXiv 2608.08081), Abstract.  The Walsh-Hadamard
transform followed by block-diagonal SO(4) rotations is there to make each
vector's coordinates statistically alike (spread outlier energy over all 128
coordinates) before the 3-bit scalar quantizer with one scale per vector.
These statistics measure that, for the method's transform and for the
variants it is compared with: no transform, the WHT alone, the SO(4) blocks
alone, and a dense rotation (16,384 parameters instead of 256).

Readings (the pages name the effect, not a measure of it):
  * per-coordinate kurtosis across the tokens: Pearson's m4 / m2^2 with
    population central moments (a Gaussian coordinate gives 3);
  * within-vector kurtosis: the same over one vector's 128 entries, averaged
    over the tokens;
  * a variance counts as zero (and its kurtosis is reported as 0) when it is
    at most 1e-9 times the mean square of the same values;
  * relative quantization error: sum of squared errors of the 3-bit quantizer
    (the one in isoquant.quantize) over sum of squares, both over all tokens
    and coordinates;
  * peak-to-average power ratio: 128 max_i y_i^2 / sum_i y_i^2 per vector,
    averaged over the vectors that are not zero.
"""
import numpy as np

from .isoquant import D, NBLK, LEVELS, HALF_RANGE, hadamard, block_matrix

TRANSFORMS = ("none", "wht", "so4", "wht_so4", "dense")
N_STATS = 260            # [0:128] kurtosis, [128:256] variance, then the four scalars below
I_VEC_KURT, I_REL_MSE, I_PAPR, I_COUNT = 256, 257, 258, 259
ZERO_VAR = 1e-9


def block_diagonal(params):
    """blockdiag(M_0..M_31) of one head's SO(4) parameters ([32][8], q_L then q_R)."""
    p = np.asarray(params, dtype=np.float64).reshape(NBLK, 8)
    B = np.zeros((D, D))
    for b in range(NBLK):
        B[4 * b:4 * b + 4, 4 * b:4 * b + 4] = block_matrix(p[b, 0:4], p[b, 4:8])
    return B


def transform_matrix(mode, params=None, dense=None):
    """The 128x128 matrix T of a transform variant, applied as y = T x."""
    if mode == "none":
        return np.eye(D)
    if mode == "wht":
        return hadamard(D)
    if mode == "so4":
        return block_diagonal(params)
    if mode == "wht_so4":                     # the method: WHT first, then the SO(4) blocks
        return block_diagonal(params) @ hadamard(D)
    if mode == "dense":
        return np.asarray(dense, dtype=np.float64).reshape(D, D)
    raise ValueError(mode)


def _kurtosis(m2, m4, mean_sq):
    ok = m2 > ZERO_VAR * mean_sq
    return np.where(ok, m4 / np.where(ok, m2 * m2, 1.0), 0.0)


def _quantize_levels(y):
    """The 3-bit quantizer of isoquant.quantize applied to already transformed rows y."""
    a = np.max(np.abs(y), axis=-1)
    s = a / HALF_RANGE
    safe = np.where(s > 0, s, 1.0)
    codes = np.clip(np.floor(y / safe[..., None] + LEVELS / 2), 0, LEVELS - 1)
    codes = np.where((s > 0)[..., None], codes, LEVELS / 2)
    return s[..., None] * (codes - HALF_RANGE)


def isotropy_stats(x, mode, params=None, dense=None):
    """Statistics of y = T x over the rows x of one head ([n_tokens][128]).

    Returns float64 [260]: per-coordinate kurtosis [0:128] and variance
    [128:256] across the tokens; then the mean within-vector kurtosis, the
    relative quantization error, the mean peak-to-average power ratio and the
    token count.  No tokens gives all zeros.
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1, D)
    out = np.zeros(N_STATS)
    n = x.shape[0]
    if n == 0:
        return out
    y = x @ transform_matrix(mode, params, dense).T
    # across the tokens, per coordinate
    c = y - y.mean(axis=0)
    m2, m4 = np.mean(c ** 2, axis=0), np.mean(c ** 4, axis=0)
    out[0:D] = _kurtosis(m2, m4, np.mean(y ** 2, axis=0))
    out[D:2 * D] = m2
    # within each vector, across its coordinates
    cv = y - y.mean(axis=1, keepdims=True)
    v2, v4 = np.mean(cv ** 2, axis=1), np.mean(cv ** 4, axis=1)
    out[I_VEC_KURT] = np.mean(_kurtosis(v2, v4, np.mean(y ** 2, axis=1)))
    # 3-bit quantization error
    energy = np.sum(y ** 2)
    err = np.sum((y - _quantize_levels(y)) ** 2)
    out[I_REL_MSE] = err / energy if energy > 0 else 0.0
    norms = np.sum(y ** 2, axis=1)
    nz = norms > 0
    out[I_PAPR] = np.mean(D * np.max(y[nz] ** 2, axis=1) / norms[nz]) if np.any(nz) else 0.0
    out[I_COUNT] = n
    return out
