"""GPU parity of multi-token attention on the packed cache
(iq_decode_attention_multi) against the oracle (multi_token_attention),
through the C ABI: ragged lengths, a sequence shorter than the number of query
tokens, fp32 queries with shared rotations, a 16-token chunk, an odd count with
several chunks per token group, more than 64 token groups, and one token,
which must be exactly iq_decode_attention.  Tolerance as for decode
(tests/_parity.py).
"""
import numpy as np
import pytest
import torch

import _parity as P
import compressed_space_decode_amd as iq
import oracle
from compressed_space_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


def _cache(rng, B, Hkv, cap, shared=False):
    k = (rng.standard_normal((B, Hkv, cap, 128)) * 1.5).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    g = rng.standard_normal(((1 if shared else B), Hkv, 32, 2, 4))
    params = (g / np.linalg.norm(g, axis=-1, keepdims=True)).reshape(-1, Hkv, 32, 8).astype(np.float32)
    rot = torch.from_numpy(params[0] if shared else params).cuda()
    kc, ks = P.empty_cache(B, Hkv, cap)
    vc, vs = P.empty_cache(B, Hkv, cap)
    iq.quantize_kv(P.torch_input(W.f32_to_bf16_bits(k), "bf16"), P.torch_input(W.f32_to_bf16_bits(v), "bf16"),
                   rot, kc, ks, vc, vs, shared_rot=shared)
    pfull = np.broadcast_to(params, (B, Hkv, 32, 8)) if shared else params
    return (kc, ks, vc, vs), rot, pfull


def _check(rng, B, Q, Hq, Hkv, cap, lens, qdtype="bf16", shared=False, what=""):
    cache, rot, params = _cache(rng, B, Hkv, cap, shared)
    q = (rng.standard_normal((B, Q, Hq, 128)) * 2.0).astype(np.float32)
    qin = W.f32_to_bf16_bits(q) if qdtype == "bf16" else q
    lens_t = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = iq.decode_attention_multi(P.torch_input(qin, qdtype), *cache, rot, seq_lens=lens_t, shared_rot=shared)
    torch.cuda.synchronize()
    kc, ks, vc, vs = [t.cpu().numpy() for t in cache]
    lens_np = np.full(B, cap) if lens is None else np.asarray(lens)
    ref = oracle.multi_token_attention(W.to_f64(qin, qdtype), oracle.unpack(kc), ks, oracle.unpack(vc), vs, params,
                                       lens_np)
    err = P.check_output(out.cpu().numpy(), ref, what=what)
    print("%s: max abs error %.3g" % (what, err), flush=True)
    return out, cache, rot, qin


def test_multi_token_ragged_lengths_and_short_sequence():
    rng = np.random.default_rng(61)
    out, *_ = _check(rng, 3, 4, 16, 2, 3000, [3000, 1234, 3], what="Q=4 ragged")
    assert torch.all(out[2, 0] == 0)                 # position -1: sees nothing
    assert not torch.all(out[2, 1] == 0)


def test_multi_token_f32_queries_shared_rotation_full_cache():
    rng = np.random.default_rng(62)
    _check(rng, 2, 3, 8, 4, 1500, None, qdtype="f32", shared=True, what="Q=3 f32 shared")


def test_multi_token_odd_count_many_chunks_and_empty_tokens():
    # Q = 5: token groups of 4 and 1 (three of the last group's tokens are absent, one of them in a
    # pair with a present token); lengths long enough for several chunks per group, and a
    # sequence of 4 whose first token sees nothing
    rng = np.random.default_rng(66)
    out, *_ = _check(rng, 3, 5, 16, 2, 2600, [2600, 700, 4], what="Q=5 ragged")
    assert torch.all(out[2, 0] == 0)                 # position -1
    assert not torch.all(out[2, 1] == 0)


def test_multi_token_more_than_64_token_groups():
    # 70 sequences of 6 tokens: 140 token groups (of 4 and 2), so the chunk plan takes its
    # 64-at-a-time path
    rng = np.random.default_rng(67)
    lens = list(rng.integers(0, 601, size=70))
    lens[3], lens[7] = 0, 2                        # an empty sequence and one shorter than Q
    out, *_ = _check(rng, 70, 6, 8, 2, 600, lens, what="Q=6 B=70")
    assert torch.all(out[3] == 0) and torch.all(out[7, :4] == 0)


def test_multi_token_chunk_of_sixteen():
    rng = np.random.default_rng(63)
    _check(rng, 1, 16, 32, 4, 4096, [4000], what="Q=16")


def test_one_token_is_decode_attention():
    rng = np.random.default_rng(64)
    out, cache, rot, qin = _check(rng, 2, 1, 8, 2, 2000, [2000, 777], what="Q=1")
    lens = torch.tensor([2000, 777], dtype=torch.int32, device="cuda")
    dec = iq.decode_attention(P.torch_input(qin[:, 0], "bf16"), *cache, rot, seq_lens=lens)
    assert torch.equal(out[:, 0], dec)


def test_multi_token_two_head_groups():
    # 16 query heads per KV head: each token's rows span two head groups
    rng = np.random.default_rng(65)
    _check(rng, 2, 2, 32, 2, 1200, [1200, 517], what="Q=2 G=16")
