"""GPU parity of the record formats (iq_quantize_kv_format,
iq_decode_attention_format) against the oracle (oracle/formats.py), through
the C ABI.

Codes: bit-exact except a fraction <= 1e-4 of one-level differences, each
next to a decision threshold (within 1e-6 of the vector's max |x'|, as for the
3-bit codes); scales within 1e-6 relative; attention outputs within max-abs
2e-3 of the oracle on the GPU's codes.  The 3-bit format through the format
entry points must equal the dedicated ones byte for byte.
"""
import numpy as np
import pytest
import torch

import _parity as P
import compressed_space_decode_amd as iq
from compressed_space_decode_amd import workloads as W
from oracle import formats as F

pytestmark = pytest.mark.gpu


def _params(rng, *lead):
    g = rng.standard_normal(lead + (32, 2, 4))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    return g.reshape(lead + (32, 8)).astype(np.float32)


def _cache(n_seq, H, cap, fmt):
    codes = torch.zeros((n_seq, H, cap, F.record_bytes(fmt)), dtype=torch.uint8, device="cuda")
    scales = torch.zeros(iq.scale_shape((n_seq, H, cap), fmt), dtype=torch.float32, device="cuda")
    return codes, scales


def _check_codes(x64, params, rec, sc, fmt, what):
    """x64 [N][128] inputs of one head; GPU records and scales."""
    b = F.bits(fmt)
    codes_o, scales_o, s_o, u = F.quantize_format(x64, params, fmt)
    codes_g = F.unpack_bits(rec, b)
    mism = codes_g != codes_o
    n = int(mism.sum())
    if n:
        rows, cols = np.nonzero(mism)
        assert np.all(np.abs(codes_g[mism].astype(int) - codes_o[mism].astype(int)) == 1), what
        if fmt == "a3":
            amax = np.full(u.shape[0], 7.0)                   # the range max x' - min x' in units of the step
        else:
            amax = np.max(np.abs(u - (2 ** (b - 1) if fmt != "lm3" else 0.0)), axis=1)   # max|x'| in step units
        if fmt == "lm3":
            L = np.array(F.LLOYD_MAX_8)
            th = (L[:-1] + L[1:]) / 2
            dist = np.min(np.abs(u[rows, cols][:, None] - th[None, :]), axis=1)
        else:
            dist = np.abs(u[rows, cols] - np.rint(u[rows, cols]))
        assert np.all(dist <= 1e-6 * amax[rows] + 1e-12), "%s: a code differs away from a threshold" % what
    if fmt == "a3":      # (s, m): the step within 1e-6 relative, the minimum within 1e-6 of the range
        np.testing.assert_allclose(sc[:, 0], scales_o[:, 0].astype(np.float64), rtol=1e-6, atol=0, err_msg=what)
        rng_ = 7.0 * scales_o[:, 0].astype(np.float64)
        assert np.all(np.abs(sc[:, 1] - scales_o[:, 1].astype(np.float64)) <= 1e-6 * rng_ + 1e-30), what
    else:
        np.testing.assert_allclose(sc, scales_o.astype(np.float64), rtol=1e-6, atol=0, err_msg=what)
    return n


@pytest.mark.parametrize("fmt", ["u2", "u4", "lm3", "a3"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_format_matches_oracle(fmt, dtype):
    rng = np.random.default_rng(200 + F.FORMATS.index(fmt) + (10 if dtype == "bf16" else 0))
    n_seq, H, T, off, cap = 2, 3, 523, 7, 540
    x = rng.standard_t(4, size=(n_seq, H, T, 128)).astype(np.float32)
    x[0, 0, 3] = 0.0                                  # a zero vector
    xin = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    params = _params(rng, n_seq, H)
    kc, ks = _cache(n_seq, H, cap, fmt)
    kc.fill_(0xAB)
    iq.quantize_kv(P.torch_input(xin, dtype), None, torch.from_numpy(params).cuda(), kc, ks, None, None,
                   tok_offset=off, fmt=fmt)
    torch.cuda.synchronize()
    rec, sc = kc.cpu().numpy(), ks.cpu().numpy()
    assert np.all(rec[:, :, :off] == 0xAB) and np.all(rec[:, :, off + T:] == 0xAB)   # nothing else written
    x64 = W.to_f64(xin, dtype)
    flips = 0
    for s_ in range(n_seq):
        for h in range(H):
            flips += _check_codes(x64[s_, h], params[s_, h], rec[s_, h, off:off + T], sc[s_, h, off:off + T], fmt,
                                  "%s %s s=%d h=%d" % (fmt, dtype, s_, h))
    assert flips <= max(1, 1e-4 * x.size)
    print("%s %s: %d threshold flips of %d codes" % (fmt, dtype, flips, x.size), flush=True)


@pytest.mark.parametrize("fmt", ["u2", "u4", "lm3", "a3"])
def test_decode_format_matches_oracle(fmt):
    rng = np.random.default_rng(220 + F.FORMATS.index(fmt))
    B, Hq, Hkv, cap = 3, 16, 2, 2100
    lens = [2100, 777, 0]
    k = (rng.standard_normal((B, Hkv, cap, 128)) * 1.5).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    q = (rng.standard_normal((B, Hq, 128)) * 2.0).astype(np.float32)
    params = _params(rng, B, Hkv)
    rot = torch.from_numpy(params).cuda()
    kc, ks = _cache(B, Hkv, cap, fmt)
    vc, vs = _cache(B, Hkv, cap, fmt)
    iq.quantize_kv(P.torch_input(W.f32_to_bf16_bits(k), "bf16"), P.torch_input(W.f32_to_bf16_bits(v), "bf16"), rot,
                   kc, ks, vc, vs, fmt=fmt)
    qin = W.f32_to_bf16_bits(q)
    out = iq.decode_attention(P.torch_input(qin, "bf16"), kc, ks, vc, vs, rot,
                              seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"), fmt=fmt)
    torch.cuda.synchronize()
    b = F.bits(fmt)
    ref = F.decode_attention_format(W.to_f64(qin, "bf16"), F.unpack_bits(kc.cpu().numpy(), b), ks.cpu().numpy(),
                                    F.unpack_bits(vc.cpu().numpy(), b), vs.cpu().numpy(), params, np.array(lens), fmt)
    err = P.check_output(out.cpu().numpy(), ref, what="decode %s" % fmt)
    assert torch.all(out[2] == 0)
    print("decode %s: max abs error %.3g" % (fmt, err), flush=True)


def test_three_bit_format_through_the_format_entry_points_is_the_dedicated_path():
    rng = np.random.default_rng(230)
    B, Hq, Hkv, cap = 2, 8, 2, 900
    x = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32))
    rot = torch.from_numpy(_params(rng, B, Hkv)).cuda()
    xt = P.torch_input(x, "bf16")
    a = P.empty_cache(B, Hkv, cap)
    c = P.empty_cache(B, Hkv, cap)
    iq.quantize_kv(xt, None, rot, a[0], a[1], None, None)
    lib = iq.lib()
    rc = lib.iq_quantize_kv_format(xt.data_ptr(), None, 1, B, Hkv, cap, xt.stride(0), xt.stride(1), xt.stride(2),
                                   rot.data_ptr(), Hkv * 256, c[0].data_ptr(), c[1].data_ptr(), None, None, cap, 0,
                                   128, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


@pytest.mark.parametrize("fmt,Hq,Hkv", [("u4", 4, 4), ("lm3", 24, 2), ("u2", 3, 1), ("a3", 12, 1)])
def test_decode_format_head_groupings(fmt, Hq, Hkv):
    # G = 1 (three of the four waves hold no head), G = 12 (two head groups, the second with four
    # heads) and G = 3
    rng = np.random.default_rng(240 + Hq)
    B, cap = 2, 700
    lens = [700, 333]
    k = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    q = (rng.standard_normal((B, Hq, 128)) * 2.0).astype(np.float32)
    params = _params(rng, B, Hkv)
    rot = torch.from_numpy(params).cuda()
    kc, ks = _cache(B, Hkv, cap, fmt)
    vc, vs = _cache(B, Hkv, cap, fmt)
    iq.quantize_kv(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), rot, kc, ks, vc, vs, fmt=fmt)
    out = iq.decode_attention(torch.from_numpy(q).cuda(), kc, ks, vc, vs, rot,
                              seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"), fmt=fmt)
    torch.cuda.synchronize()
    b = F.bits(fmt)
    ref = F.decode_attention_format(q.astype(np.float64), F.unpack_bits(kc.cpu().numpy(), b), ks.cpu().numpy(),
                                    F.unpack_bits(vc.cpu().numpy(), b), vs.cpu().numpy(), params, np.array(lens), fmt)
    P.check_output(out.cpu().numpy(), ref, what="decode %s Hq=%d Hkv=%d" % (fmt, Hq, Hkv))


@pytest.mark.parametrize("fmt", ["lm3", "u2", "u4"])
def test_decode_format_on_uniformly_random_records(fmt):
    # Random record bytes: every code value at every field position of K and V (3-bit fields that
    # straddle bytes included), so each operand plane and each unpack mask meets every pattern.
    # Scales are small so the scores stay moderate; the second sequence ends in a partial block.
    rng = np.random.default_rng(240 + F.FORMATS.index(fmt))
    B, Hq, Hkv, cap = 2, 8, 2, 1400
    lens = [1400, 613]
    rb = F.record_bytes(fmt)
    kc = torch.from_numpy(rng.integers(0, 256, (B, Hkv, cap, rb), dtype=np.uint8)).cuda()
    vc = torch.from_numpy(rng.integers(0, 256, (B, Hkv, cap, rb), dtype=np.uint8)).cuda()
    ks = torch.from_numpy((rng.random((B, Hkv, cap)) * 0.2 + 0.02).astype(np.float32)).cuda()
    vs = torch.from_numpy((rng.random((B, Hkv, cap)) * 0.5 + 0.05).astype(np.float32)).cuda()
    params = _params(rng, B, Hkv)
    rot = torch.from_numpy(params).cuda()
    q = (rng.standard_normal((B, Hq, 128)) * 2.0).astype(np.float32)
    qin = W.f32_to_bf16_bits(q)
    out = iq.decode_attention(P.torch_input(qin, "bf16"), kc, ks, vc, vs, rot,
                              seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"), fmt=fmt)
    torch.cuda.synchronize()
    b = F.bits(fmt)
    ref = F.decode_attention_format(W.to_f64(qin, "bf16"), F.unpack_bits(kc.cpu().numpy(), b), ks.cpu().numpy(),
                                    F.unpack_bits(vc.cpu().numpy(), b), vs.cpu().numpy(), params, np.array(lens), fmt)
    err = P.check_output(out.cpu().numpy(), ref, what="decode %s, random records" % fmt)
    print("decode %s on random records: max abs error %.3g" % (fmt, err), flush=True)
