"""Seeded synthetic workloads (inputs only: no step of the method lives here).

Both the HIP path and the CPU oracle take their inputs from this module, so
it holds only random-number draws and dtype rounding.  Shapes and value
distributions follow the five workloads the hot path is measured on:

  tiny     B=1,  Hq=4,  Hkv=4, T=512,   fp32, Q/K/V ~ N(0,1)
  gqa8k    B=1,  Hq=32, Hkv=4, T=8192,  bf16, K ~ N(0,1) with 4 channels per
           KV head scaled x20, V ~ N(0,1), Q ~ N(0,1)
  prefill  48 layers x Hkv=4 x T=32768, bf16, K and V ~ Student-t (nu = 3),
           quantization only (generated one layer at a time)
  long32k  B=1,  Hq=32, Hkv=4, T=32768, bf16, K[t,h,c] = sigma[h,c] z with
           sigma log-uniform on [0.1, 30], V, Q ~ N(0,1), one planted key
           K[p,h,:] = 4 Q[h G,:] per KV head at a seeded position p
  ragged   B=16, Hq=32, Hkv=8, cap 32768, per-sequence lengths uniform on
           [1024, 32768], Q/K/V ~ N(0,1), 2% of K elements set to +-25

Recipe: workload i uses numpy SeedSequence(i) spawned into child streams
(rotation, Q, K, V, extra); K and V are drawn per sequence from children of
their stream so sequences can be drawn in parallel threads.  Normal draws
are float32 (numpy's float32 generator); Student-t(3) is z / sqrt(2 g / 3)
with z ~ N(0,1) and g ~ Gamma(1.5, 1), both float32.  bf16 values are the
float32 draws rounded to nearest even.  Rotation parameters: per (layer or
sequence, KV head) 32 blocks of a left and a right unit quaternion, each a
normalised N(0, I_4) draw (uniform on the 3-sphere), stored float32.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

WORKLOAD_IDS = {"tiny": 1, "gqa8k": 2, "prefill": 3, "long32k": 4, "ragged": 5}
SHAPES = {   # B, Hq, Hkv, T, dtype
    "tiny": (1, 4, 4, 512, "f32"),
    "gqa8k": (1, 32, 4, 8192, "bf16"),
    "long32k": (1, 32, 4, 32768, "bf16"),
    "ragged": (16, 32, 8, 32768, "bf16"),
}
PREFILL_SHAPE = (48, 4, 32768)   # layers, Hkv, T
D = 128
_THREADS = 8


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (nearest even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def rotation_params(rng, n):
    """float32 [n][32][8] unit quaternion pairs (normalised Gaussian draws)."""
    g = rng.standard_normal((n, 32, 2, 4))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    return g.reshape(n, 32, 8).astype(np.float32)


def dense_rotations(seed, n):
    """float32 [n][128][128] random rotations for the dense-rotation comparison: Haar-distributed
    orthogonal matrices (QR of a Gaussian matrix with the signs of R's diagonal moved into Q),
    drawn from SeedSequence([6, seed])."""
    rng = np.random.default_rng(np.random.SeedSequence([6, int(seed)]))
    a = rng.standard_normal((n, D, D))
    q, r = np.linalg.qr(a)
    return (q * np.sign(np.diagonal(r, axis1=-2, axis2=-1))[:, None, :]).astype(np.float32)


def multi_token_queries(n_seq, n_tokens, n_q_heads):
    """bf16 bits [n_seq][n_tokens][n_q_heads][128]: N(0,1) queries of several new tokens per
    sequence, drawn from SeedSequence([7, n_tokens])."""
    rng = np.random.default_rng(np.random.SeedSequence([7, int(n_tokens)]))
    return f32_to_bf16_bits(rng.standard_normal((n_seq, n_tokens, n_q_heads, D), dtype=np.float32))


def _as_dtype(x, dtype):
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return np.asarray(x, dtype=np.float32)


def _student_t3(rng, shape):
    z = rng.standard_normal(size=shape, dtype=np.float32)
    g = rng.standard_gamma(1.5, size=shape, dtype=np.float32)
    return z / np.sqrt(g * np.float32(2.0 / 3.0))


def _per_seq(parent_seq, B, fn):
    kids = parent_seq.spawn(B)
    with ThreadPoolExecutor(_THREADS) as ex:
        return list(ex.map(lambda i: fn(i, np.random.default_rng(kids[i])), range(B)))


def decode_workload(workload, tokens=None, batch=None):
    """Inputs for one of the decode workloads (tiny, gqa8k, long32k, ragged).

    ``tokens`` / ``batch`` shrink the workload for quick tests while keeping
    its distributions.  Returns a dict with
      q [B][Hq][128], k, v [B][Hkv][T][128]  (uint16 bf16 bits or float32),
      dtype ("f32" | "bf16"), params float32 [B][Hkv][32][8],
      seq_lens int32 [B], n_q_heads, n_kv_heads, and for long32k the planted
      position per sequence.
    """
    B, Hq, Hkv, T, dtype = SHAPES[workload]
    if tokens is not None:
        T = int(tokens)
    if batch is not None:
        B = int(batch)
    G = Hq // Hkv
    s_rot, s_q, s_k, s_v, s_x = np.random.SeedSequence(WORKLOAD_IDS[workload]).spawn(5)
    r_x = np.random.default_rng(s_x)
    params = rotation_params(np.random.default_rng(s_rot), B * Hkv).reshape(B, Hkv, 32, 8)
    q = _as_dtype(np.random.default_rng(s_q).standard_normal((B, Hq, D), dtype=np.float32), dtype)
    q32 = bf16_bits_to_f32(q) if dtype == "bf16" else q
    seq_lens = np.full(B, T, dtype=np.int32)
    extra = {}
    chans = sigma = pos = None
    if workload == "gqa8k":
        chans = np.stack([np.stack([r_x.choice(D, size=4, replace=False) for _ in range(Hkv)]) for _ in range(B)])
    elif workload == "long32k":
        sigma = np.exp(r_x.uniform(np.log(0.1), np.log(30.0), size=(B, Hkv, D))).astype(np.float32)
        pos = r_x.integers(0, T, size=B)
        extra["planted_pos"] = pos.astype(np.int64)
    elif workload == "ragged":
        seq_lens = r_x.integers(min(1024, T), T + 1, size=B).astype(np.int32)

    def gen_k(b, rng):
        k = rng.standard_normal((Hkv, T, D), dtype=np.float32)
        if workload == "gqa8k":
            for h in range(Hkv):
                k[h][:, chans[b, h]] *= np.float32(20.0)
        elif workload == "long32k":
            k *= sigma[b][:, None, :]
            for h in range(Hkv):
                k[h, pos[b], :] = np.float32(4.0) * q32[b, h * G, :]
        elif workload == "ragged":
            hit = rng.random((Hkv, T, D), dtype=np.float32) < np.float32(0.02)
            neg = rng.random((Hkv, T, D), dtype=np.float32) < np.float32(0.5)
            k = np.where(hit, np.where(neg, np.float32(-25.0), np.float32(25.0)), k)
        return _as_dtype(k, dtype)

    def gen_v(b, rng):
        return _as_dtype(rng.standard_normal((Hkv, T, D), dtype=np.float32), dtype)

    k = np.stack(_per_seq(s_k, B, gen_k))
    v = np.stack(_per_seq(s_v, B, gen_v))
    return dict(workload=workload, q=q, k=k, v=v, dtype=dtype, params=params,
                seq_lens=seq_lens, n_q_heads=Hq, n_kv_heads=Hkv, **extra)


def prefill_layer(layer, tokens=PREFILL_SHAPE[2], n_kv_heads=PREFILL_SHAPE[1]):
    """One layer of the bulk-prefill workload: (k, v) uint16 bf16 bits
    [Hkv][T][128] drawn Student-t (nu = 3), and params float32 [Hkv][32][8].
    Each layer has its own child seeds so any layer can be regenerated alone."""
    s_rot, s_k, s_v = np.random.SeedSequence([WORKLOAD_IDS["prefill"], int(layer)]).spawn(3)
    params = rotation_params(np.random.default_rng(s_rot), n_kv_heads)
    k = _student_t3(np.random.default_rng(s_k), (n_kv_heads, tokens, D))
    v = _student_t3(np.random.default_rng(s_v), (n_kv_heads, tokens, D))
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v), params


def prefill_layers(layers, tokens=PREFILL_SHAPE[2], n_kv_heads=PREFILL_SHAPE[1]):
    """Several prefill layers drawn in parallel threads (same values as prefill_layer)."""
    with ThreadPoolExecutor(_THREADS) as ex:
        return list(ex.map(lambda l: prefill_layer(l, tokens, n_kv_heads), layers))


def to_f64(x, dtype):
    """Exact conversion of a workload array to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
