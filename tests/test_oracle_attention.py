"""Pins for the oracle's compressed-space decode attention.

Pages: "RotaryQuant ..." (arXiv 2608.08081), Abstract -- attention runs
directly on the packed 3-bit tensors without materialising full-precision
KV.  Pinned by the orthogonality identity (compressed space equals dense
attention on dequantized, unrotated K/V), by PyTorch's fp64 scaled-dot-
product attention on tiny cases, and by closed-form special cases.
"""
import numpy as np
import pytest
import torch

import oracle


def _case(rng, B=2, Hq=4, Hkv=2, T=37, lens=None):
    p = rng.standard_normal((B, Hkv, 32, 2, 4))
    p /= np.linalg.norm(p, axis=-1, keepdims=True)
    p = p.reshape(B, Hkv, 32, 8)
    q = rng.standard_normal((B, Hq, 128))
    k = rng.standard_normal((B, Hkv, T, 128)) * 2.0
    v = rng.standard_normal((B, Hkv, T, 128))
    kc = np.zeros((B, Hkv, T, 128), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((B, Hkv, T), np.float32)
    vs = np.zeros_like(ks)
    for b in range(B):
        for g in range(Hkv):
            kc[b, g], ks[b, g], _, _ = oracle.quantize(k[b, g], p[b, g])
            vc[b, g], vs[b, g], _, _ = oracle.quantize(v[b, g], p[b, g])
    if lens is None:
        lens = np.full(B, T)
    return q, kc, ks, vc, vs, p, np.asarray(lens)


def test_compressed_space_equals_dense_on_dequantized():
    rng = np.random.default_rng(20)
    args = _case(rng, lens=[37, 11])
    a = oracle.decode_attention(*args)
    b = oracle.dense_attention_on_dequantized(*args)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(21)
    q, kc, ks, vc, vs, p, lens = _case(rng, B=1, Hq=6, Hkv=3, T=19)
    out = oracle.decode_attention(q, kc, ks, vc, vs, p, lens)
    G = 2
    for g in range(3):
        R = oracle.rotation_matrix(p[0, g])
        khat = torch.tensor(oracle.dequantize_rotated(kc[0, g], ks[0, g]) @ R)
        vhat = torch.tensor(oracle.dequantize_rotated(vc[0, g], vs[0, g]) @ R)
        for h in range(g * G, (g + 1) * G):
            qq = torch.tensor(q[0, h])[None, None, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, khat[None, None], vhat[None, None])[0, 0, 0].numpy()
            np.testing.assert_allclose(out[0, h], ref, rtol=1e-10, atol=1e-12)


def test_gqa_mapping_uses_contiguous_groups():
    # Query head h must read KV head h // G (contiguous groups).  KV head 0 gets every V code 7
    # (rotated-space level +3.5 s) and KV head 1 every code 0 (-3.5 s): rotating an output back
    # into its KV head's space gives a vector of one sign, telling which KV head it read.
    rng = np.random.default_rng(22)
    q, kc, ks, vc, vs, p, lens = _case(rng, B=1, Hq=4, Hkv=2, T=5)
    vc[0, 0] = 7
    vc[0, 1] = 0
    out = oracle.decode_attention(q, kc, ks, vc, vs, p, lens)
    for h in range(4):
        g = h // 2
        rot = oracle.rotation_matrix(p[0, g]) @ out[0, h]
        expect = np.sum(vs[0, g]) / 5 * 3.5   # mean scale is an upper bound; check sign and constancy
        assert np.all(rot > 0) if g == 0 else np.all(rot < 0)
        assert np.ptp(rot) < 1e-12 * expect


def test_single_token_returns_its_value():
    rng = np.random.default_rng(23)
    q, kc, ks, vc, vs, p, _ = _case(rng, B=1, Hq=2, Hkv=1, T=4)
    out = oracle.decode_attention(q, kc, ks, vc, vs, p, np.array([1]))
    R = oracle.rotation_matrix(p[0, 0])
    ref = R.T @ oracle.dequantize_rotated(vc[0, 0, 0], vs[0, 0, 0])
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-13)
    np.testing.assert_allclose(out[0, 1], ref, atol=1e-13)


def test_zero_query_gives_mean_and_zero_length_gives_zero():
    rng = np.random.default_rng(24)
    q, kc, ks, vc, vs, p, _ = _case(rng, B=2, Hq=2, Hkv=1, T=9)
    q[:] = 0
    out = oracle.decode_attention(q, kc, ks, vc, vs, p, np.array([9, 0]))
    R = oracle.rotation_matrix(p[0, 0])
    ref = R.T @ oracle.dequantize_rotated(vc[0, 0], vs[0, 0]).mean(axis=0)
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-13)
    assert np.all(out[1] == 0)


def test_softmax_scale_default_and_override():
    rng = np.random.default_rng(25)
    args = list(_case(rng, B=1, Hq=1, Hkv=1, T=8))
    a = oracle.decode_attention(*args, sm_scale=None)
    b = oracle.decode_attention(*args, sm_scale=1 / np.sqrt(128))
    c = oracle.decode_attention(*args, sm_scale=0.5)
    np.testing.assert_array_equal(a, b)
    assert np.max(np.abs(a - c)) > 1e-6


def test_split_merge_equals_two_pass():
    # Online split-K merge (max, rescale, sum) reproduces the two-pass softmax: this is the
    # identity the combine step relies on.
    rng = np.random.default_rng(26)
    z = rng.standard_normal(100) * 5
    v = rng.standard_normal((100, 128))
    p = np.exp(z - z.max())
    ref = (p @ v) / p.sum()
    parts = []
    for lo in range(0, 100, 17):
        zz = z[lo:lo + 17]
        m = zz.max()
        w = np.exp(zz - m)
        parts.append((m, w.sum(), w @ v[lo:lo + 17]))
    M = max(m for m, _, _ in parts)
    L = sum(np.exp(m - M) * l for m, l, _ in parts)
    O = sum(np.exp(m - M) * o for m, _, o in parts)
    np.testing.assert_allclose(O / L, ref, atol=1e-13)


def test_retrieval_of_a_planted_key_survives_quantization_in_oracle():
    # Small analogue of the long-context planted-key workload: the planted position wins
    # the softmax after 3-bit quantization.
    rng = np.random.default_rng(27)
    T = 2048
    p = rng.standard_normal((1, 1, 32, 2, 4))
    p /= np.linalg.norm(p, axis=-1, keepdims=True)
    p = p.reshape(1, 1, 32, 8)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, T, 128))
    pos = 777
    k[0, 0, pos] = 4 * q[0, 0]
    kc, ks, _, _ = oracle.quantize(k[0, 0], p[0, 0])
    R = oracle.rotation_matrix(p[0, 0])
    z = oracle.dequantize_rotated(kc, ks) @ (R @ q[0, 0])
    assert int(np.argmax(z)) == pos


def test_long32k_planted_key_retrieval_exact_and_3bit_in_oracle():
    # The long-context workload at full size (one layer: 4 KV heads x 32768 tokens), the oracle's
    # own codes: per KV head, the argmax of the exact fp64 scores q.k and of the 3-bit scores
    # (R q).k_hat for the query head the key was planted for.  3-bit quantization keeps every head
    # the exact scores retrieve; the exact scores miss KV head 0, where another key's
    # channel-scaled score is higher than the planted key's before any quantization.
    from compressed_space_decode_amd import workloads as W
    w = W.decode_workload("long32k")
    p = int(w["planted_pos"][0])
    q64 = W.to_f64(w["q"], w["dtype"])
    G = w["n_q_heads"] // w["n_kv_heads"]
    exact, packed = [], []
    for h in range(w["n_kv_heads"]):
        k64 = W.to_f64(w["k"][0, h], w["dtype"])
        qh = q64[0, h * G]
        codes, scales, _, _ = oracle.quantize(k64, w["params"][0, h])
        R = oracle.rotation_matrix(w["params"][0, h])
        exact.append(int(np.argmax(k64 @ qh)) == p)
        packed.append(int(np.argmax(oracle.dequantize_rotated(codes, scales) @ (R @ qh))) == p)
    assert exact == [False, True, True, True]
    assert packed == exact


def test_multi_token_attention_matches_masked_torch_sdpa():
    # Q new tokens at the last Q positions, each attending to the positions up to its own:
    # PyTorch's fp64 attention with an explicit boolean mask on the dequantized, unrotated K/V.
    rng = np.random.default_rng(30)
    T, Q = 23, 4
    _, kc, ks, vc, vs, p, _ = _case(rng, B=2, Hq=4, Hkv=2, T=T)
    q = rng.standard_normal((2, Q, 4, 128))
    lens = np.array([T, 15])
    out = oracle.multi_token_attention(q, kc, ks, vc, vs, p, lens)
    for b in range(2):
        n = lens[b]
        mask = torch.tensor(np.arange(T)[None, :] <= (n - Q + np.arange(Q))[:, None])
        for g in range(2):
            R = oracle.rotation_matrix(p[b, g])
            khat = torch.tensor(oracle.dequantize_rotated(kc[b, g], ks[b, g]) @ R)
            vhat = torch.tensor(oracle.dequantize_rotated(vc[b, g], vs[b, g]) @ R)
            for h in range(2 * g, 2 * g + 2):
                qq = torch.tensor(q[b, :, h])[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, khat[None, None], vhat[None, None], attn_mask=mask)[0, 0].numpy()
                np.testing.assert_allclose(out[b, :, h], ref, rtol=1e-10, atol=1e-12)


def test_multi_token_attention_special_cases():
    rng = np.random.default_rng(31)
    q1, kc, ks, vc, vs, p, lens = _case(rng, B=2, Hq=4, Hkv=2, T=20, lens=[20, 9])
    # one query token is a decode step
    one = oracle.multi_token_attention(q1[:, None], kc, ks, vc, vs, p, lens)
    np.testing.assert_array_equal(one[:, 0], oracle.decode_attention(q1, kc, ks, vc, vs, p, lens))
    # a token never sees later positions: changing them leaves it unchanged
    Q = 3
    q = rng.standard_normal((2, Q, 4, 128))
    base = oracle.multi_token_attention(q, kc, ks, vc, vs, p, lens)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, :, 19] = 7 - kc2[0, :, 19]                 # the last position: only the last token sees it
    vc2[0, :, 19] = 7 - vc2[0, :, 19]
    moved = oracle.multi_token_attention(q, kc2, ks, vc2, vs, p, lens)
    np.testing.assert_array_equal(moved[0, :Q - 1], base[0, :Q - 1])
    assert not np.allclose(moved[0, Q - 1], base[0, Q - 1])
    # positions below zero (a sequence shorter than Q) see nothing
    short = oracle.multi_token_attention(q, kc, ks, vc, vs, p, np.array([2, 9]))
    assert np.all(short[0, 0] == 0) and np.any(short[0, 1] != 0)
