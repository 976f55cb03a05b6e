"""IsoQuant oracle, fp64, written step by step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function follows
"RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
Compressed-Space Attention" (arXiv 2608.08081), Abstract, plus the readings
stated in each docstring where that text is silent.

Notation: d = 128 coordinates per head vector, 32 blocks of 4 coordinates,
3-bit codes (8 levels), one fp32 scale per vector, 48-byte packed records.
"""
import numpy as np

D = 128                 # head dimension
NBLK = D // 4           # number of SO(4) blocks
LEVELS = 8              # 3-bit codes
RECORD_BYTES = D * 3 // 8   # 48 bytes of packed codes per vector
HALF_RANGE = LEVELS / 2 - 0.5   # 3.5: outermost level magnitude in units of s


# --------------------------------------------------------------------------
# Input conversion
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits):
    """Exact bf16 -> fp64: a bf16 value is the top 16 bits of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Walsh-Hadamard transform (Abstract: the first stage of the rotation)
# --------------------------------------------------------------------------
def hadamard(n=D):
    """Normalised Sylvester-order Hadamard matrix, H[i, j] = (-1)^popcount(i & j) / sqrt(n).

    Reading: natural (Sylvester) ordering, no random sign diagonal, and the
    1/sqrt(n) normalisation that makes H orthogonal (and its own inverse).
    Built densely: this is the O(d^2) definition, not a fast transform.
    """
    i = np.arange(n)
    parity = np.zeros((n, n), dtype=np.int64)
    x = i[:, None] & i[None, :]
    while np.any(x):
        parity ^= (x & 1)
        x = x >> 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(n)


# --------------------------------------------------------------------------
# SO(4) blocks from a left/right unit-quaternion pair
# (Abstract: the second stage, 4x4 rotation blocks on the diagonal, 256 stored parameters
# per head)
# --------------------------------------------------------------------------
def quat_left(a):
    """4x4 matrix of v -> a * v (Hamilton product, components (w, x, y, z))."""
    a0, a1, a2, a3 = a
    return np.array([[a0, -a1, -a2, -a3],
                     [a1, a0, -a3, a2],
                     [a2, a3, a0, -a1],
                     [a3, -a2, a1, a0]], dtype=np.float64)


def quat_right(b):
    """4x4 matrix of v -> v * b (Hamilton product)."""
    b0, b1, b2, b3 = b
    return np.array([[b0, -b1, -b2, -b3],
                     [b1, b0, b3, -b2],
                     [b2, -b3, b0, b1],
                     [b3, b2, -b1, b0]], dtype=np.float64)


def quat_conj(r):
    r = np.asarray(r, dtype=np.float64)
    return np.array([r[0], -r[1], -r[2], -r[3]])


def block_matrix(q_left, q_right):
    """The SO(4) block v -> q_L * v * conj(q_R) as a 4x4 matrix.

    Reading: each block holds one left and one right quaternion (8 numbers;
    32 blocks x 8 = 256 parameters per head).  Both quaternions are
    normalised in fp64 before use, so the block is exactly orthogonal with
    determinant +1 whatever rounding the stored parameters carry.
    """
    ql = np.asarray(q_left, dtype=np.float64)
    qr = np.asarray(q_right, dtype=np.float64)
    ql = ql / np.sqrt(np.dot(ql, ql))
    qr = qr / np.sqrt(np.dot(qr, qr))
    return quat_left(ql) @ quat_right(quat_conj(qr))


def rotation_matrix(params):
    """Dense 128x128 rotation R = blockdiag(M_0..M_31) @ H for one head.

    ``params`` is [32][8]: params[b, 0:4] = q_L, params[b, 4:8] = q_R of
    block b, which acts on coordinates 4b..4b+3.  Order: WHT first, then
    the block rotation (Abstract: the Walsh-Hadamard stage, then the diagonal of
    SO(4) blocks).
    """
    p = np.asarray(params, dtype=np.float64).reshape(NBLK, 8)
    B = np.zeros((D, D))
    for b in range(NBLK):
        B[4 * b:4 * b + 4, 4 * b:4 * b + 4] = block_matrix(p[b, 0:4], p[b, 4:8])
    return B @ hadamard(D)


def rotate(x, params):
    """x' = R x for every row of x (shape [..., 128])."""
    R = rotation_matrix(params)
    return np.asarray(x, dtype=np.float64) @ R.T


# --------------------------------------------------------------------------
# 3-bit scalar quantization with a per-vector scale
# (Abstract: each coordinate of the rotated vector gets a 3-bit scalar code)
# --------------------------------------------------------------------------
def quantize(x, params):
    """Rotate, then quantize each 128-vector to 3-bit codes and one fp32 scale.

    Reading (symmetric uniform mid-rise quantizer): a = max|x'|,
    s = a / 3.5, code = clamp(floor(x'/s + 4), 0, 7); the level of code c is
    s * (c - 3.5).  floor sends a value on a threshold to the upper code.
    a == 0 gives s = 0 and every code 4.  The decision is taken in fp64 on
    the fp64 rotated value; the stored scale is s rounded to fp32.

    Returns (codes uint8 [..., 128], scales float32 [...], x_rot float64
    [..., 128], s_exact float64 [...]); the last two let tests measure how
    close each coordinate is to a decision threshold.
    """
    xr = rotate(x, params)
    a = np.max(np.abs(xr), axis=-1)
    s = a / HALF_RANGE
    safe = np.where(s > 0, s, 1.0)
    u = xr / safe[..., None] + LEVELS / 2
    codes = np.clip(np.floor(u), 0, LEVELS - 1)
    codes = np.where((s > 0)[..., None], codes, LEVELS / 2)
    return codes.astype(np.uint8), s.astype(np.float32), xr, s


def dequantize_rotated(codes, scales):
    """Levels in rotated space: s * (c - 3.5), fp64."""
    return (np.asarray(scales, np.float64)[..., None]
            * (np.asarray(codes, np.float64) - HALF_RANGE))


# --------------------------------------------------------------------------
# Bit layout of a 48-byte record (Abstract: the cache holds the codes packed at
# 3 bits each; the layout itself is a reading).
#
# The 128 codes form one little-endian bit stream of 384 bits: bit b of the
# code of coordinate i is stream bit 3i + b, and byte k of the record holds
# stream bits 8k..8k+7 (bit 8k + m is bit m of byte k).  Equivalently, every
# 3 bytes 3g..3g+2 hold the 8 codes of coordinates 8g..8g+7 as the 24-bit
# little-endian number sum_j c_(8g+j) 8^j.
# --------------------------------------------------------------------------
def pack(codes):
    """uint8 codes [..., 128] (values 0..7) -> uint8 records [..., 48]."""
    c = np.asarray(codes)
    assert c.shape[-1] == D and np.all(c < LEVELS)
    c = c.astype(np.uint8)
    lead = c.shape[:-1]
    bits = np.zeros(lead + (3 * D,), dtype=np.uint8)        # the stream, one entry per bit
    for i in range(D):
        for b in range(3):
            bits[..., 3 * i + b] = (c[..., i] >> b) & 1
    out = np.zeros(lead + (RECORD_BYTES,), dtype=np.uint8)
    for k in range(RECORD_BYTES):
        for m in range(8):
            out[..., k] |= bits[..., 8 * k + m] << m
    return out


def unpack(records):
    """uint8 records [..., 48] -> uint8 codes [..., 128]; inverse of pack."""
    r = np.asarray(records, dtype=np.uint8)
    assert r.shape[-1] == RECORD_BYTES
    lead = r.shape[:-1]
    bits = np.zeros(lead + (3 * D,), dtype=np.uint8)
    for k in range(RECORD_BYTES):
        for m in range(8):
            bits[..., 8 * k + m] = (r[..., k] >> m) & 1
    codes = np.zeros(lead + (D,), dtype=np.uint8)
    for i in range(D):
        for b in range(3):
            codes[..., i] |= bits[..., 3 * i + b] << b
    return codes


# --------------------------------------------------------------------------
# Decode attention on packed codes (Abstract: attention runs on the packed codes;
# no full-precision K/V is ever formed).
# --------------------------------------------------------------------------
def decode_attention(q, k_codes, k_scales, v_codes, v_scales, params, seq_lens,
                     sm_scale=None):
    """One decode step in the compressed space, two-pass softmax, fp64.

    Shapes: q [B][Hq][128]; k_codes/v_codes uint8 [B][Hkv][T][128] (unpacked
    codes); k_scales/v_scales [B][Hkv][T]; params [B][Hkv][32][8] (one
    rotation per (sequence or layer, KV head), shared by K and V);
    seq_lens [B].  Returns float64 [B][Hq][128].

    Readings: query head h reads KV head h // (Hq/Hkv); tokens t < len are
    all visible; sm_scale defaults to 1/sqrt(128).  Because R is orthogonal,
    q.k_hat = (Rq).(s(c - 3.5)) with k_hat the unrotated dequantized key, so
    the query is rotated once, the weighted sum of V levels is formed in
    rotated space and rotated back once per output: o = R^T o'.  len = 0
    gives a zero output.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_codes.shape[1]
    assert d == D and Hq % Hkv == 0
    G = Hq // Hkv
    sm = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        for g in range(Hkv):
            R = rotation_matrix(params[b][g])
            kq = dequantize_rotated(k_codes[b, g, :n], k_scales[b, g, :n])
            vq = dequantize_rotated(v_codes[b, g, :n], v_scales[b, g, :n])
            for h in range(g * G, (g + 1) * G):
                qr = R @ q[b, h]
                z = sm * (kq @ qr)
                m = np.max(z)
                p = np.exp(z - m)
                o_rot = (p @ vq) / np.sum(p)
                out[b, h] = R.T @ o_rot
    return out


def multi_token_attention(q, k_codes, k_scales, v_codes, v_scales, params, seq_lens,
                          sm_scale=None):
    """Attention of several new query tokens per sequence on the packed cache, fp64.

    Shapes: q [B][Q][Hq][128]; the cache as in decode_attention; seq_lens [B]
    counts the cached tokens including the Q new ones, which are the last Q
    positions.  Returns float64 [B][Q][Hq][128].

    Reading (the paper's execution model applied to more than one query, as
    in chunked prefill or checking several drafted tokens at once): query
    token i of sequence b sits at position seq_lens[b] - Q + i and attends
    causally to positions 0 .. seq_lens[b] - Q + i; a token whose position is
    below 0 sees nothing and gets zeros.  Each token's result is a decode
    step with that length.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Q = q.shape[:2]
    out = np.zeros(q.shape)
    for i in range(Q):
        lens = np.maximum(np.asarray(seq_lens, dtype=np.int64) - Q + i + 1, 0)
        out[:, i] = decode_attention(q[:, i], k_codes, k_scales, v_codes, v_scales, params, lens,
                                     sm_scale=sm_scale)
    return out


def dense_attention_on_dequantized(q, k_codes, k_scales, v_codes, v_scales, params,
                                   seq_lens, sm_scale=None):
    """The same attention computed the conventional way: dequantize K and V,
    rotate them back to the original space, then plain softmax attention with
    the unrotated query.  Equal to decode_attention up to fp64 rounding
    because R is orthogonal; tests use it as a cross-check."""
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
            k_hat = dequantize_rotated(k_codes[b, g, :n], k_scales[b, g, :n]) @ R
            v_hat = dequantize_rotated(v_codes[b, g, :n], v_scales[b, g, :n]) @ R
            for h in range(g * G, (g + 1) * G):
                z = sm * (k_hat @ q[b, h])
                w = np.exp(z - z.max())
                out[b, h] = (w / w.sum()) @ v_hat
    return out
