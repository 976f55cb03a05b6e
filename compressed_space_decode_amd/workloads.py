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

Rotation parameters: per (layer or sequence, KV head), 32 blocks of a left
and a right unit quaternion, each drawn as a normalised N(0, I_4) vector
(uniform on the 3-sphere), stored fp32.

Seeds: workload i uses numpy SeedSequence(i) spawned into independent child
streams in the order (rotation, Q, K, V, extra); bf16 values are produced by
rounding the fp64 draw to fp32 and then to bf16, both to nearest even.
"""
import numpy as np

WORKLOAD_IDS = {"tiny": 1, "gqa8k": 2, "prefill": 3, "long32k": 4, "ragged": 5}
D = 128


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (nearest even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def rotation_params(rng, n):
    """float32 [n][32][8] unit quaternion pairs (normalised Gaussian draws)."""
    g = rng.standard_normal((n, 32, 2, 4))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    return g.reshape(n, 32, 8).astype(np.float32)


def _streams(workload, n=5):
    ss = np.random.SeedSequence(WORKLOAD_IDS[workload])
    return [np.random.default_rng(s) for s in ss.spawn(n)]


def _as_dtype(x, dtype):
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    return x.astype(np.float32)


def decode_workload(workload, tokens=None, batch=None):
    """Inputs for one of the decode workloads (tiny, gqa8k, long32k, ragged).

    ``tokens`` / ``batch`` shrink the workload for quick tests while keeping
    its distributions.  Returns a dict with
      q [B][Hq][128], k, v [B][Hkv][T][128]  (uint16 bf16 bits or float32),
      dtype ("f32" | "bf16"), params float32 [B][Hkv][32][8],
      seq_lens int32 [B], n_q_heads, n_kv_heads, and for long32k the planted
      position per sequence.
    """
    r_rot, r_q, r_k, r_v, r_x = _streams(workload)
    if workload == "tiny":
        B, Hq, Hkv, T, dtype = 1, 4, 4, 512, "f32"
    elif workload == "gqa8k":
        B, Hq, Hkv, T, dtype = 1, 32, 4, 8192, "bf16"
    elif workload == "long32k":
        B, Hq, Hkv, T, dtype = 1, 32, 4, 32768, "bf16"
    elif workload == "ragged":
        B, Hq, Hkv, T, dtype = 16, 32, 8, 32768, "bf16"
    else:
        raise ValueError(workload)
    if tokens is not None:
        T = int(tokens)
    if batch is not None:
        B = int(batch)
    G = Hq // Hkv
    params = rotation_params(r_rot, B * Hkv).reshape(B, Hkv, 32, 8)
    q = r_q.standard_normal((B, Hq, D))
    k = r_k.standard_normal((B, Hkv, T, D))
    v = r_v.standard_normal((B, Hkv, T, D))
    seq_lens = np.full(B, T, dtype=np.int32)
    extra = {}
    if workload == "gqa8k":
        for b in range(B):
            for h in range(Hkv):
                ch = r_x.choice(D, size=4, replace=False)
                k[b, h, :, ch] *= 20.0
    elif workload == "long32k":
        sigma = np.exp(r_x.uniform(np.log(0.1), np.log(30.0), size=(B, Hkv, D)))
        k *= sigma[:, :, None, :]
        pos = r_x.integers(0, T, size=B)
        qb = _as_dtype(q, dtype)
        qf = bf16_bits_to_f32(qb).astype(np.float64) if dtype == "bf16" else qb.astype(np.float64)
        for b in range(B):
            for h in range(Hkv):
                k[b, h, pos[b], :] = 4.0 * qf[b, h * G, :]
        extra["planted_pos"] = pos.astype(np.int64)
    elif workload == "ragged":
        lo = min(1024, T)
        seq_lens = r_x.integers(lo, T + 1, size=B).astype(np.int32)
        hit = r_x.random(k.shape) < 0.02
        sign = np.where(r_x.random(k.shape) < 0.5, -1.0, 1.0)
        k = np.where(hit, 25.0 * sign, k)
    return dict(workload=workload, q=_as_dtype(q, dtype), k=_as_dtype(k, dtype),
                v=_as_dtype(v, dtype), dtype=dtype, params=params,
                seq_lens=seq_lens, n_q_heads=Hq, n_kv_heads=Hkv, **extra)


def prefill_layer(layer, tokens=32768, n_kv_heads=4):
    """One layer of the bulk-prefill workload: (k, v) uint16 bf16 bits
    [Hkv][T][128] drawn Student-t (nu = 3), and params float32 [Hkv][32][8].
    Each layer has its own child seed so any layer can be regenerated alone."""
    ss = np.random.SeedSequence([WORKLOAD_IDS["prefill"], int(layer)])
    r_rot, r_k, r_v = [np.random.default_rng(s) for s in ss.spawn(3)]
    params = rotation_params(r_rot, n_kv_heads)
    k = r_k.standard_t(3, size=(n_kv_heads, tokens, D)).astype(np.float32)
    v = r_v.standard_t(3, size=(n_kv_heads, tokens, D)).astype(np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v), params


def to_f64(x, dtype):
    """Exact conversion of a workload array to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
