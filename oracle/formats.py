"""Bit-width and codebook variants of the scalar quantizer, and attention on them (fp64).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing on the product
path imports it, and it shares no code with the HIP path.

Source: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
Compressed-Space Attention" (arXiv 2608.08081), Abstract: after the rotation
the vectors go through 3-bit scalar quantization and are stored packed.  The
variants here keep the rotation and change only the quantizer.  Every function
is pinned by tests/test_oracle_formats.py.

Readings (the pages fix only "3-bit scalar"):
  * "u2", "u3", "u4": symmetric uniform mid-rise quantizer with 2^b levels and
    one scale per vector, s = max|x'| / (2^(b-1) - 1/2),
    code = clamp(floor(x'/s + 2^(b-1)), 0, 2^b - 1), level s (c - (2^b - 1)/2).
    "u3" is isoquant.quantize.  A zero vector gives s = 0 and code 2^(b-1).
  * "lm3": the 8-level Lloyd-Max quantizer of a unit Gaussian, with the levels
    J. Max printed ("Quantizing for minimum distortion", 1960): 0.2451, 0.7560,
    1.344, 2.152 and their negatives.  They are scaled by the vector's RMS
    sigma = |x'| / sqrt(128): the code is the number of midpoints between consecutive levels that are at or below
    x'/sigma (the nearest level, ties upward) and the value is sigma L[c].
    A zero vector gives sigma = 0 and code 4.  The stored scale is sigma.
  * "a3": the asymmetric (min/max) alternative to the symmetric 3-bit quantizer,
    as in the KIVI-style schemes the pages cite: the 8 levels are equally spaced
    from the vector's minimum m to its maximum M, s = (M - m) / 7,
    code = clamp(floor((x' - m)/s + 1/2), 0, 7) (the nearest level, ties upward),
    value m + s c.  A constant vector gives s = 0 and code 0 (value m, exact).
    Two numbers are stored per vector, (s, m): its scales array has a trailing
    dimension of 2.  Its records are the 3-bit records of "u3".
  * Records: one little-endian bit stream of b bits per code (bit j of code i
    is stream bit b*i + j, byte k holds stream bits 8k..8k+7): 16 b bytes.
"""
import math

import numpy as np

from .isoquant import D, rotate, rotation_matrix

FORMATS = ("u2", "u3", "u4", "lm3", "a3")
LLOYD_MAX_8 = (-2.152, -1.344, -0.7560, -0.2451, 0.2451, 0.7560, 1.344, 2.152)   # as Max printed them


def bits(fmt):
    return {"u2": 2, "u3": 3, "u4": 4, "lm3": 3, "a3": 3}[fmt]


def scale_words(fmt):
    """fp32 numbers stored per vector: (s, m) for "a3", one scale otherwise."""
    return 2 if fmt == "a3" else 1


def record_bytes(fmt):
    return 16 * bits(fmt)


def pack_bits(codes, b):
    """uint8 codes [..., 128] (values < 2^b) -> uint8 records [..., 16 b]."""
    c = np.asarray(codes).astype(np.uint8)
    assert c.shape[-1] == D and np.all(c < (1 << b))
    lead = c.shape[:-1]
    stream = np.zeros(lead + (b * D,), dtype=np.uint8)
    for i in range(D):
        for j in range(b):
            stream[..., b * i + j] = (c[..., i] >> j) & 1
    out = np.zeros(lead + (16 * b,), dtype=np.uint8)
    for k in range(16 * b):
        for m in range(8):
            out[..., k] |= stream[..., 8 * k + m] << m
    return out


def unpack_bits(records, b):
    """uint8 records [..., 16 b] -> uint8 codes [..., 128]; inverse of pack_bits."""
    r = np.asarray(records, dtype=np.uint8)
    assert r.shape[-1] == 16 * b
    lead = r.shape[:-1]
    stream = np.zeros(lead + (b * D,), dtype=np.uint8)
    for k in range(16 * b):
        for m in range(8):
            stream[..., 8 * k + m] = (r[..., k] >> m) & 1
    codes = np.zeros(lead + (D,), dtype=np.uint8)
    for i in range(D):
        for j in range(b):
            codes[..., i] |= stream[..., b * i + j] << j
    return codes


def quantize_rotated(y, fmt):
    """Quantize rows y [..., 128] that are already rotated.  Returns (codes uint8,
    scales float32, s_exact float64, u float64): u is the value compared with the
    decision thresholds (x'/s + 2^(b-1) for the uniform formats, x'/sigma for lm3,
    (x' - m)/s + 1/2 for a3), so that tests can measure how close a decision was.
    For a3 the scales have a trailing dimension of 2: (s, m)."""
    y = np.asarray(y, dtype=np.float64)
    if fmt == "a3":
        m = np.min(y, axis=-1)
        s = (np.max(y, axis=-1) - m) / 7.0
        safe = np.where(s > 0, s, 1.0)
        u = (y - m[..., None]) / safe[..., None] + 0.5
        codes = np.clip(np.floor(u), 0, 7)
        codes = np.where((s > 0)[..., None], codes, 0)
        return codes.astype(np.uint8), np.stack([s, m], axis=-1).astype(np.float32), s, u
    if fmt == "lm3":
        sigma = np.sqrt(np.sum(y * y, axis=-1) / D)
        safe = np.where(sigma > 0, sigma, 1.0)
        u = y / safe[..., None]
        L = np.array(LLOYD_MAX_8)
        mids = (L[:-1] + L[1:]) / 2
        codes = np.zeros(y.shape, dtype=np.int64)
        for t in mids:
            codes += (u >= t)
        codes = np.where((sigma > 0)[..., None], codes, 4)
        return codes.astype(np.uint8), sigma.astype(np.float32), sigma, u
    b = bits(fmt)
    half = 2 ** (b - 1)
    s = np.max(np.abs(y), axis=-1) / (half - 0.5)
    safe = np.where(s > 0, s, 1.0)
    u = y / safe[..., None] + half
    codes = np.clip(np.floor(u), 0, 2 ** b - 1)
    codes = np.where((s > 0)[..., None], codes, half)
    return codes.astype(np.uint8), s.astype(np.float32), s, u


def quantize_format(x, params, fmt):
    """Rotate (isoquant.rotate), then quantize in format fmt."""
    return quantize_rotated(rotate(x, params), fmt)


def levels(codes, scales, fmt):
    """Values in rotated space of codes [..., 128] with their per-vector scales, fp64."""
    c = np.asarray(codes, dtype=np.int64)
    if fmt == "a3":
        sm = np.asarray(scales, dtype=np.float64)
        return sm[..., 1:2] + sm[..., 0:1] * c
    sc = np.asarray(scales, dtype=np.float64)[..., None]
    if fmt == "lm3":
        return sc * np.array(LLOYD_MAX_8)[c]
    b = bits(fmt)
    return sc * (c - (2 ** b - 1) / 2.0)


def decode_attention_format(q, k_codes, k_scales, v_codes, v_scales, params, seq_lens, fmt,
                            sm_scale=None):
    """decode_attention on a cache of format fmt (unpacked codes), fp64, two-pass softmax.
    Same readings as isoquant.decode_attention: head h reads KV head h // (Hq/Hkv), scores
    q.k_hat = (Rq).level(k), o = R^T sum p level(v) / sum p, length 0 gives zeros."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    sm = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        for g in range(Hkv):
            R = rotation_matrix(params[b][g])
            kq = levels(k_codes[b, g, :n], k_scales[b, g, :n], fmt)
            vq = levels(v_codes[b, g, :n], v_scales[b, g, :n], fmt)
            for h in range(g * G, (g + 1) * G):
                z = sm * (kq @ (R @ q[b, h]))
                p = np.exp(z - np.max(z))
                out[b, h] = R.T @ ((p @ vq) / np.sum(p))
    return out


def lloyd_max_gaussian(n_levels, iters=2000):
    """Lloyd's fixed point for a unit Gaussian source: thresholds at the midpoints of
    consecutive levels, each level the conditional mean of its cell,
    E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  fp64."""
    phi = lambda t: 0.0 if math.isinf(t) else math.exp(-0.5 * t * t) / math.sqrt(2 * math.pi)
    Phi = lambda t: 0.5 * (1.0 + math.erf(t / math.sqrt(2.0)))
    L = np.linspace(-2.0, 2.0, n_levels)
    for _ in range(iters):
        edges = [-math.inf] + list((L[:-1] + L[1:]) / 2) + [math.inf]
        L = np.array([(phi(a) - phi(b)) / (Phi(b) - Phi(a)) for a, b in zip(edges[:-1], edges[1:])])
    return L


def gaussian_distortion(levels_):
    """Mean squared error of a quantizer with the given levels (nearest level) on a unit
    Gaussian, by exact integration: sum over cells of E[(X - L)^2; cell]."""
    L = np.asarray(levels_, dtype=np.float64)
    edges = [-math.inf] + list((L[:-1] + L[1:]) / 2) + [math.inf]
    phi = lambda t: 0.0 if math.isinf(t) else math.exp(-0.5 * t * t) / math.sqrt(2 * math.pi)
    Phi = lambda t: 0.5 * (1.0 + math.erf(t / math.sqrt(2.0)))
    tphi = lambda t: 0.0 if math.isinf(t) else t * phi(t)
    total = 0.0
    for (a, b), c in zip(zip(edges[:-1], edges[1:]), L):
        p = Phi(b) - Phi(a)
        m1 = phi(a) - phi(b)                       # E[X; cell]
        m2 = p + tphi(a) - tphi(b)                 # E[X^2; cell]
        total += m2 - 2 * c * m1 + c * c * p
    return total
