"""GPU tests of the fused append + decode entry point (iq_decode_attention_append)
through the C ABI.

The fused call must leave the cache byte-for-byte as iq_quantize_kv of the new
token would, and return what iq_decode_attention returns on that cache with
lengths positions + 1; both are also checked against the CPU oracle
(tolerances in tests/_parity.py).  Positions are ragged, include the first and
last cache slots and chunk boundaries, and out-of-range positions skip their
sequence.
"""
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


def _setup(rng, B, Hq, Hkv, cap, dtype="bf16", shared=False):
    """A filled cache (every position quantised from random K/V), new K/V vectors and queries."""
    k = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    k_new = (rng.standard_normal((B, Hkv, 128)) * 3.0).astype(np.float32)
    v_new = rng.standard_normal((B, Hkv, 128)).astype(np.float32)
    q = (rng.standard_normal((B, Hq, 128)) * 2.0).astype(np.float32)
    params = _params(rng, 1 if shared else B, Hkv)
    cvt = (lambda x: W.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    rot = torch.from_numpy(params[0] if shared else params).cuda()
    kc, ks = P.empty_cache(B, Hkv, cap)
    vc, vs = P.empty_cache(B, Hkv, cap)
    iq.quantize_kv(P.torch_input(cvt(k), dtype), P.torch_input(cvt(v), dtype), rot, kc, ks, vc, vs,
                   shared_rot=shared)
    pfull = np.broadcast_to(params, (B, Hkv, 32, 8)) if shared else params
    return dict(k_new=cvt(k_new), v_new=cvt(v_new), q=cvt(q), dtype=dtype, rot=rot, params=pfull,
                cache=(kc, ks, vc, vs), shared=shared)


def _two_call(s, positions, cap):
    """Reference on the GPU: quantize_kv of each sequence's token at its position, then decode."""
    kc, ks, vc, vs = [t.clone() for t in s["cache"]]
    B = kc.shape[0]
    kn, vn = P.torch_input(s["k_new"], s["dtype"]), P.torch_input(s["v_new"], s["dtype"])
    for b in range(B):
        p = int(positions[b])
        if 0 <= p < cap:
            rot_b = s["rot"] if s["shared"] else s["rot"][b:b + 1]
            iq.quantize_kv(kn[b:b + 1, :, None], vn[b:b + 1, :, None], rot_b, kc[b:b + 1], ks[b:b + 1],
                           vc[b:b + 1], vs[b:b + 1], tok_offset=p, shared_rot=s["shared"])
    lens = torch.tensor([p + 1 if 0 <= p < cap else 0 for p in positions], dtype=torch.int32, device="cuda")
    out = iq.decode_attention(P.torch_input(s["q"], s["dtype"]), kc, ks, vc, vs, s["rot"], seq_lens=lens,
                              shared_rot=s["shared"])
    torch.cuda.synchronize()
    return out, (kc, ks, vc, vs)


def _fused(s, positions, workspace=None):
    kc, ks, vc, vs = [t.clone() for t in s["cache"]]
    pos = torch.tensor(positions, dtype=torch.int32, device="cuda")
    out = iq.decode_attention_append(P.torch_input(s["q"], s["dtype"]), P.torch_input(s["k_new"], s["dtype"]),
                                     P.torch_input(s["v_new"], s["dtype"]), pos, kc, ks, vc, vs, s["rot"],
                                     workspace=workspace, shared_rot=s["shared"])
    torch.cuda.synchronize()
    return out, (kc, ks, vc, vs)


def _check(s, positions, cap, what, workspace=None):
    out_f, cache_f = _fused(s, positions, workspace)
    out_r, cache_r = _two_call(s, positions, cap)
    for a, b, name in zip(cache_f, cache_r, ("k codes", "k scales", "v codes", "v scales")):
        assert torch.equal(a, b), "%s: fused append left different %s" % (what, name)
    diff = float((out_f - out_r).abs().max())
    assert diff <= 1e-6, "%s: fused vs two-call output differs by %.3g" % (what, diff)
    # oracle: the new token's codes, then attention on the resulting cache
    kc, ks, vc, vs = [t.cpu().numpy() for t in cache_f]
    for b, p in enumerate(positions):
        if not 0 <= p < cap:
            continue
        for h in range(kc.shape[1]):
            for side, rec, sc in (("k_new", kc, ks), ("v_new", vc, vs)):
                x64 = W.to_f64(s[side][b, h][None], s["dtype"])
                n, _ = P.check_quantize(x64, s["params"][b, h], rec[b, h, p][None], sc[b, h, p][None],
                                        what="%s %s b=%d h=%d" % (what, side, b, h))
                assert n <= 1
    lens = np.array([p + 1 if 0 <= p < cap else 0 for p in positions])
    ref = oracle.decode_attention(W.to_f64(s["q"], s["dtype"]), oracle.unpack(kc), ks, oracle.unpack(vc), vs,
                                  s["params"], lens)
    err = P.check_output(out_f.cpu().numpy(), ref, what=what)
    print("%s: max abs error %.3g" % (what, err), flush=True)
    return out_f


def test_append_ragged_positions_match_two_call_path_and_oracle():
    rng = np.random.default_rng(41)
    cap = 3000
    s = _setup(rng, 4, 16, 2, cap)
    _check(s, [0, 1234, cap - 1, 1023], cap, "ragged positions")


def test_append_at_chunk_boundaries_with_two_head_groups():
    # 16 query heads per KV head: two work-groups (head groups) share each chunk and both write
    # the new token's records.
    rng = np.random.default_rng(42)
    cap = 4096
    s = _setup(rng, 3, 32, 2, cap)
    _check(s, [127, 128, 2559], cap, "chunk boundaries, G=16")


def test_append_out_of_range_positions_skip_the_sequence():
    rng = np.random.default_rng(43)
    cap = 700
    s = _setup(rng, 3, 8, 2, cap)
    out = _check(s, [-1, cap, 5], cap, "out-of-range positions")
    assert torch.all(out[:2] == 0)


def test_append_f32_inputs_and_shared_rotation():
    rng = np.random.default_rng(44)
    cap = 2000
    s = _setup(rng, 2, 12, 3, cap, dtype="f32", shared=True)
    _check(s, [1999, 640], cap, "f32, shared rotation")


def test_append_inside_and_after_the_first_blocks_of_a_chunk():
    # Each wave loads its chunk's first two 32-token blocks before the query set-up; the
    # work-group whose first 256 tokens hold the new token loads them only after the append.
    # With these lengths the kernels pick 512-token chunks (640 at three work-groups per compute
    # unit, on 256 compute units): position 2600 is token 40 of its chunk (loaded after the
    # append), 5520 is token 400 of its chunk (past the early blocks), 300 is in the first chunk,
    # 8191 is the last slot.
    rng = np.random.default_rng(45)
    cap = 8192
    s = _setup(rng, 8, 8, 8, cap)
    positions = [2600, 5520, 300, 8000, 8000, 8000, 8000, cap - 1]
    ws = torch.zeros(iq.decode_workspace_bytes(8, 8, 8, cap), dtype=torch.uint8, device="cuda")
    _check(s, positions, cap, "append in and past the early blocks", workspace=ws)
    chunk = int(ws[:4].view(torch.int32)[0])          # the plan at the start of the workspace
    offsets = [p % chunk for p in positions]
    assert any(p >= chunk and o < 256 for p, o in zip(positions, offsets)), (chunk, offsets)
    assert any(o >= 256 for o in offsets), (chunk, offsets)
