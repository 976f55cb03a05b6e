"""GPU test of a decode loop captured once as a HIP graph and replayed: each
replay runs iq_decode_attention_append on static buffers whose contents (query,
new K/V, positions) the host changes between replays.

Every replay must leave the cache byte-for-byte as the same call made eagerly
does, and return the same output; the last step is also checked against the
CPU oracle (tolerances in tests/_parity.py).  The library records no memset
and allocates nothing inside the call, so the graph holds only its two kernels.
"""
import numpy as np
import pytest
import torch

import _parity as P
import compressed_space_decode_amd as iq
import oracle
from compressed_space_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_graph_replayed_decode_loop_matches_eager_calls():
    rng = np.random.default_rng(51)
    B, Hq, Hkv, cap, steps = 3, 16, 2, 2048, 5
    start = np.array([700, 1279, cap - steps + 1])       # the last sequence runs past the cache end
    g = rng.standard_normal((B, Hkv, 32, 2, 4))
    params = (g / np.linalg.norm(g, axis=-1, keepdims=True)).reshape(B, Hkv, 32, 8).astype(np.float32)
    rot = torch.from_numpy(params).cuda()
    hist_k = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32))
    hist_v = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32))
    kc, ks = P.empty_cache(B, Hkv, cap)
    vc, vs = P.empty_cache(B, Hkv, cap)
    iq.quantize_kv(P.torch_input(hist_k, "bf16"), P.torch_input(hist_v, "bf16"), rot, kc, ks, vc, vs)
    eager = [t.clone() for t in (kc, ks, vc, vs)]

    # static buffers the graph reads and writes
    q_s = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    kn_s = torch.zeros((B, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    vn_s = torch.zeros_like(kn_s)
    pos_s = torch.full((B,), -1, dtype=torch.int32, device="cuda")     # nothing appended while capturing
    out_s = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(iq.decode_workspace_bytes(B, Hq, Hkv, cap), dtype=torch.uint8, device="cuda")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                        # warm-up call off the capture
        iq.decode_attention_append(q_s, kn_s, vn_s, pos_s, kc, ks, vc, vs, rot, out=out_s, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        iq.decode_attention_append(q_s, kn_s, vn_s, pos_s, kc, ks, vc, vs, rot, out=out_s, workspace=ws)
    torch.cuda.synchronize()

    for i in range(steps):
        q = W.f32_to_bf16_bits((rng.standard_normal((B, Hq, 128)) * 2.0).astype(np.float32))
        kn = W.f32_to_bf16_bits((rng.standard_normal((B, Hkv, 128)) * 3.0).astype(np.float32))
        vn = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, 128)).astype(np.float32))
        pos = (start + i).astype(np.int32)
        q_t, kn_t, vn_t = (P.torch_input(x, "bf16") for x in (q, kn, vn))
        pos_t = torch.from_numpy(pos).cuda()
        q_s.copy_(q_t)
        kn_s.copy_(kn_t)
        vn_s.copy_(vn_t)
        pos_s.copy_(pos_t)
        graph.replay()
        # eager call on its own cache copy, with a fresh workspace
        out_e = iq.decode_attention_append(q_t, kn_t, vn_t, pos_t, *eager, rot)
        torch.cuda.synchronize()
        for a, b, name in zip((kc, ks, vc, vs), eager, ("k codes", "k scales", "v codes", "v scales")):
            assert torch.equal(a, b), "replay %d left different %s" % (i, name)
        assert torch.equal(out_s, out_e), "replay %d output differs from the eager call" % i
        print("replay %d: positions %s, output equal to the eager call" % (i, pos.tolist()), flush=True)

    # the last replay against the oracle; the last sequence's position is past the cache: zeros
    assert pos[-1] >= cap and torch.all(out_s[-1] == 0)
    lens = np.where(pos < cap, pos + 1, 0)
    codes_k, codes_v = oracle.unpack(kc.cpu().numpy()), oracle.unpack(vc.cpu().numpy())
    ref = oracle.decode_attention(W.to_f64(q, "bf16"), codes_k, ks.cpu().numpy(), codes_v, vs.cpu().numpy(),
                                  params, lens)
    err = P.check_output(out_s.cpu().numpy(), ref, what="graph replay")
    print("last replay vs oracle: max abs error %.3g" % err, flush=True)
