"""GPU edge cases through the C ABI: ragged tails, offsets, one-token appends,
degenerate vectors, strided and partial inputs, zero/one-token sequences,
several head groupings and query dtypes.  Each is compared with the oracle
(tolerances in tests/_parity.py)."""
import numpy as np
import pytest
import torch

import _parity as P
import compressed_space_decode_amd as iq
import oracle
from compressed_space_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


def _params(rng, *lead):
    g = rng.standard_normal(lead + (32, 2, 4))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    return g.reshape(lead + (32, 8)).astype(np.float32)


def _check_all(x64, params, rec, sc, what, bound_fraction=True):
    flips, total = 0, 0
    for s in range(x64.shape[0]):
        for h in range(x64.shape[1]):
            n, _ = P.check_quantize(x64[s, h], params[s, h], rec[s, h], sc[s, h], what="%s s=%d h=%d" % (what, s, h))
            flips += n
            total += x64[s, h].size
    if bound_fraction:
        assert flips <= max(1, P.FLIP_FRACTION * total)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_ragged_tail_offset_and_untouched_cache(dtype):
    rng = np.random.default_rng(5)
    n_seq, H, T, off, cap = 2, 3, 777, 5, 800
    x = rng.standard_normal((n_seq, H, T, 128)).astype(np.float32)
    xin = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    params = _params(rng, n_seq, H)
    kc, ks = P.empty_cache(n_seq, H, cap, poison=True)
    iq.quantize_kv(P.torch_input(xin, dtype), None, torch.from_numpy(params).cuda(), kc, ks, None, None, tok_offset=off)
    torch.cuda.synchronize()
    rec, sc = kc.cpu().numpy(), ks.cpu().numpy()
    assert np.all(rec[:, :, :off] == 0xFF) and np.all(rec[:, :, off + T:] == 0xFF)
    assert np.all(sc[:, :, :off] == np.float32(1e30)) and np.all(sc[:, :, off + T:] == np.float32(1e30))
    _check_all(W.to_f64(xin, dtype), params, rec[:, :, off:off + T], sc[:, :, off:off + T], "tail")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_k_and_v_together_match_each_alone(dtype):
    # one call with both sides interleaves K and V vectors in the kernel's loop; the K-only and
    # V-only calls take the one-side path.  Ragged token count (not a multiple of 32 or 256).
    rng = np.random.default_rng(12)
    n_seq, H, T, cap = 2, 3, 301, 320
    k = rng.standard_normal((n_seq, H, T, 128)).astype(np.float32)
    v = rng.standard_normal((n_seq, H, T, 128)).astype(np.float32) * 3.0
    if dtype == "bf16":
        k, v = W.f32_to_bf16_bits(k), W.f32_to_bf16_bits(v)
    params = _params(rng, n_seq, H)
    rot = torch.from_numpy(params).cuda()
    kt, vt = P.torch_input(k, dtype), P.torch_input(v, dtype)
    kc, ks = P.empty_cache(n_seq, H, cap, poison=True)
    vc, vs = P.empty_cache(n_seq, H, cap, poison=True)
    iq.quantize_kv(kt, vt, rot, kc, ks, vc, vs, tok_offset=7)
    kc1, ks1 = P.empty_cache(n_seq, H, cap, poison=True)
    vc1, vs1 = P.empty_cache(n_seq, H, cap, poison=True)
    iq.quantize_kv(kt, None, rot, kc1, ks1, None, None, tok_offset=7)
    iq.quantize_kv(None, vt, rot, None, None, vc1, vs1, tok_offset=7)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc1) and torch.equal(ks, ks1)
    assert torch.equal(vc, vc1) and torch.equal(vs, vs1)
    rec, sc = vc.cpu().numpy(), vs.cpu().numpy()
    assert np.all(rec[:, :, :7] == 0xFF) and np.all(rec[:, :, 7 + T:] == 0xFF)
    _check_all(W.to_f64(v, dtype), params, rec[:, :, 7:7 + T], sc[:, :, 7:7 + T], "V " + dtype)


def test_quantize_one_token_appends_match_bulk():
    rng = np.random.default_rng(6)
    H, T = 2, 40
    x = W.f32_to_bf16_bits(rng.standard_normal((1, H, T, 128)).astype(np.float32))
    params = torch.from_numpy(_params(rng, 1, H)).cuda()
    xt = P.torch_input(x, "bf16")
    kc1, ks1 = P.empty_cache(1, H, T)
    iq.quantize_kv(xt, None, params, kc1, ks1, None, None)
    kc2, ks2 = P.empty_cache(1, H, T)
    for t in range(T):
        iq.quantize_kv(xt[:, :, t:t + 1], None, params, kc2, ks2, None, None, tok_offset=t)
    torch.cuda.synchronize()
    assert torch.equal(kc1, kc2) and torch.equal(ks1, ks2)


def test_quantize_degenerate_vectors():
    rng = np.random.default_rng(7)
    p = _params(rng, 1, 1)
    H128 = oracle.hadamard(128)
    R = oracle.rotation_matrix(p[0, 0])
    rows = [np.zeros(128), np.full(128, 1e-30), np.eye(128)[3] * 1e6, -np.eye(128)[100]]
    # inputs whose rotated values sit on levels, and on decision thresholds (up to fp32 input rounding)
    for vals in ([3.5, -3.5, 2.5, -0.5, 0.5], [3.5, 0.0, 1.0, -2.0, 3.0]):
        xr = np.zeros(128)
        xr[:len(vals)] = vals
        rows.append(R.T @ xr)
    x = np.stack(rows).astype(np.float32)[None, None]
    kc, ks = P.empty_cache(1, 1, x.shape[2])
    iq.quantize_kv(P.torch_input(x, "f32"), None, torch.from_numpy(p).cuda(), kc, ks, None, None)
    torch.cuda.synchronize()
    rec, sc = kc.cpu().numpy(), ks.cpu().numpy()
    assert sc[0, 0, 0] == 0 and np.all(oracle.unpack(rec[0, 0, 0]) == 4)
    # rows built to sit on thresholds may flip: each flip must still be a one-level flip
    # next to a threshold, but the random-data bound on their fraction does not apply here
    _check_all(W.to_f64(x, "f32"), p, rec, sc, "degenerate", bound_fraction=False)
    del H128


def test_quantize_strided_input_and_shared_rotation():
    rng = np.random.default_rng(8)
    big = rng.standard_normal((2, 3, 50, 256)).astype(np.float32)
    x = torch.from_numpy(big).cuda()[:, :, 3:43, 64:192]          # strides (38400, 12800, 256, 1)
    p = _params(rng, 1, 3)
    kc, ks = P.empty_cache(2, 3, 40)
    iq.quantize_kv(x, None, torch.from_numpy(p[0]).cuda(), kc, ks, None, None, shared_rot=True)
    torch.cuda.synchronize()
    x64 = big[:, :, 3:43, 64:192].astype(np.float64)
    _check_all(x64, np.stack([p[0], p[0]]), kc.cpu().numpy(), ks.cpu().numpy(), "strided")


def test_quantize_zero_tokens_is_noop():
    kc, ks = P.empty_cache(1, 1, 8, poison=True)
    x = torch.zeros((1, 1, 0, 128), dtype=torch.float32, device="cuda")
    rot = torch.zeros((1, 1, 32, 8), dtype=torch.float32, device="cuda")
    iq.quantize_kv(x, None, rot, kc, ks, None, None)
    torch.cuda.synchronize()
    assert torch.all(kc == 0xFF)


def _decode_case(rng, B, Hq, Hkv, cap, lens, qdtype="bf16", sm=0.0, shared=False, workspace=None):
    k = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32) * 1.5
    v = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32) * 2.0
    params = _params(rng, 1 if shared else B, Hkv)
    rot = torch.from_numpy(params[0] if shared else params).cuda()
    kc, ks = P.empty_cache(B, Hkv, cap)
    vc, vs = P.empty_cache(B, Hkv, cap)
    kin = W.f32_to_bf16_bits(k)
    vin = W.f32_to_bf16_bits(v)
    iq.quantize_kv(P.torch_input(kin, "bf16"), P.torch_input(vin, "bf16"),
                   rot, kc, ks, vc, vs, shared_rot=shared)
    qin = W.f32_to_bf16_bits(q) if qdtype == "bf16" else q
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = iq.decode_attention(P.torch_input(qin, qdtype), kc, ks, vc, vs, rot, seq_lens=lens_t, sm_scale=sm,
                              shared_rot=shared, workspace=workspace)
    torch.cuda.synchronize()
    pfull = np.broadcast_to(params, (B, Hkv, 32, 8)) if shared else params
    ref = oracle.decode_attention(W.to_f64(qin, qdtype), oracle.unpack(kc.cpu().numpy()), ks.cpu().numpy(),
                                  oracle.unpack(vc.cpu().numpy()), vs.cpu().numpy(), pfull, np.array(lens),
                                  sm_scale=sm if sm > 0 else None)
    return out.cpu().numpy(), ref


@pytest.mark.parametrize("lens", [[0, 1, 33, 127], [129, 2049, 300, 5000], [5000, 5000, 4999, 4097]])
def test_decode_ragged_lengths_including_empty(lens):
    rng = np.random.default_rng(sum(lens))
    out, ref = _decode_case(rng, 4, 8, 2, 5000, lens)
    P.check_output(out, ref, "lens=%s" % lens)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(out[b] == 0)


@pytest.mark.parametrize("Hq,Hkv", [(16, 1), (4, 2), (3, 3), (24, 2), (8, 8)])
def test_decode_head_groupings(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    out, ref = _decode_case(rng, 2, Hq, Hkv, 700, [700, 431])
    P.check_output(out, ref, "Hq=%d Hkv=%d" % (Hq, Hkv))


def test_decode_f32_query_softmax_scale_and_shared_rotation():
    rng = np.random.default_rng(11)
    out, ref = _decode_case(rng, 3, 8, 4, 600, [600, 1, 257], qdtype="f32", sm=0.3, shared=True)
    P.check_output(out, ref, "f32 q")


def test_decode_single_token_is_its_value():
    rng = np.random.default_rng(12)
    out, ref = _decode_case(rng, 1, 4, 1, 64, [1])
    P.check_output(out, ref, "len=1")


def test_decode_workspace_reused_across_calls():
    # One workspace (never cleared, initially garbage) serves consecutive calls of different
    # lengths, including an empty sequence: nothing from an earlier call leaks into a later one.
    rng = np.random.default_rng(31)
    B, Hq, Hkv, cap = 3, 16, 2, 6000
    ws = torch.full((iq.decode_workspace_bytes(B, Hq, Hkv, cap),), 0x7F, dtype=torch.uint8, device="cuda")
    for lens in ([6000, 3000, 17], [1, 0, 5999], [4096, 4097, 128]):
        out, ref = _decode_case(rng, B, Hq, Hkv, cap, lens, workspace=ws)
        P.check_output(out, ref, what="workspace reuse lens=%s" % lens)


@pytest.mark.parametrize("B,Hq,Hkv,cap,zero_frac", [
    (16, 32, 8, 5000, 0.0),     # ragged: the chunk size is searched for, one round of work-groups
    (70, 8, 2, 700, 0.2),       # more than 64 sequences, a fifth of them empty
    (100, 64, 2, 300, 0.0),     # more sequences than work items per column: one chunk per sequence
])
def test_decode_chunk_plan_over_ragged_batches(B, Hq, Hkv, cap, zero_frac):
    # The kernels size the chunks from the lengths; every (sequence, chunk) pair must be covered
    # exactly once, so each sequence's output matches the oracle.
    rng = np.random.default_rng(B * 1000 + cap)
    lens = rng.integers(1, cap + 1, size=B)
    lens[rng.random(B) < zero_frac] = 0
    lens[0] = cap
    out, ref = _decode_case(rng, B, Hq, Hkv, cap, [int(n) for n in lens])
    P.check_output(out, ref, "chunk plan B=%d Hq=%d Hkv=%d cap=%d" % (B, Hq, Hkv, cap))
    assert np.all(out[lens == 0] == 0)


def test_decode_at_the_largest_capacity():
    # cache_cap = 83,886,016, the largest the C ABI accepts: one (sequence, head) slice holds 4 GB of
    # K codes, so the kernels' 32-bit buffer offsets reach their limit.  Every position holds one
    # background token; the last one (written by iq_quantize_kv at that offset) a planted token whose
    # score is about ln(cap) above the background's.  Attention over every position is then the
    # closed-form mixture of the two dequantized values, weighted by multiplicity; without the last
    # position it is the background value.
    cap = 83886016
    rng = np.random.default_rng(100)      # the planted token carries about 43% of the weight
    params = _params(rng, 1, 1)
    rot = torch.from_numpy(params).cuda()
    q = rng.standard_normal(128)
    kbg, vbg, vp = rng.standard_normal(128), rng.standard_normal(128), rng.standard_normal(128) * 3.0
    sm = 1.0 / np.sqrt(128)
    kp = q / np.linalg.norm(q) * (np.log(cap) / sm / np.linalg.norm(q)) + 0.2 * kbg   # ~ln(cap) above
    small = lambda x: torch.from_numpy(np.asarray(x, np.float32).reshape(1, 1, 1, 128)).cuda()
    kc, ks = P.empty_cache(1, 1, cap)
    vc, vs = P.empty_cache(1, 1, cap)
    one = [P.empty_cache(1, 1, 1) for _ in range(2)]
    iq.quantize_kv(small(kbg), small(vbg), rot, one[0][0], one[0][1], one[1][0], one[1][1])
    kc[0, 0] = one[0][0][0, 0, 0]                         # the background record everywhere
    ks[0, 0] = one[0][1][0, 0, 0]
    vc[0, 0] = one[1][0][0, 0, 0]
    vs[0, 0] = one[1][1][0, 0, 0]
    iq.quantize_kv(small(kp), small(vp), rot, kc, ks, vc, vs, tok_offset=cap - 1)
    qt = torch.from_numpy(q.astype(np.float32).reshape(1, 1, 128)).cuda()
    outs = [iq.decode_attention(qt, kc, ks, vc, vs, rot, seq_lens=torch.tensor([n], dtype=torch.int32, device="cuda"))
            for n in (cap, cap - 1)]
    torch.cuda.synchronize()
    recs = {name: (oracle.unpack(c[0, 0, t].cpu().numpy()[None])[0], float(s[0, 0, t]))
            for name, c, s, t in (("kbg", kc, ks, 0), ("vbg", vc, vs, 0), ("kp", kc, ks, cap - 1), ("vp", vc, vs, cap - 1))}
    del kc, vc, ks, vs
    R = oracle.rotation_matrix(params[0, 0])
    deq = {n: R.T @ (s * (c.astype(np.float64) - 3.5)) for n, (c, s) in recs.items()}   # unrotated K and V hats
    z_bg, z_p = sm * q @ deq["kbg"], sm * q @ deq["kp"]
    w_bg, w_p = (cap - 1) * np.exp(z_bg - z_p), 1.0
    expect = (w_bg * deq["vbg"] + w_p * deq["vp"]) / (w_bg + w_p)
    assert 0.1 < w_p / (w_bg + w_p) < 0.9, "the planted token should carry a real share of the weight"
    P.check_output(outs[0].cpu().numpy()[0], expect[None], what="largest capacity, all positions")
    P.check_output(outs[1].cpu().numpy()[0], deq["vbg"][None], what="largest capacity, last position excluded")
