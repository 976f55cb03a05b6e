"""iq_decode_attention_noalloc (the entry point for callers that cannot allocate) against
iq_decode_attention with a caller's workspace: the same kernels on the same inputs, so the outputs
must agree bit for bit.  Two calls in a row, the second with a smaller problem, so the second reuses
the library's scratch after the first left it full of partials; then a size the scratch cannot hold
is refused before anything is launched."""
import numpy as np
import pytest
import torch

import _parity as P
import compressed_space_decode_amd as iq
import oracle
from compressed_space_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hkv, cap, lens):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    params = W.rotation_params(rng, B * Hkv).reshape(B, Hkv, 32, 8)
    rot = torch.from_numpy(params).cuda()
    kc, ks = P.empty_cache(B, Hkv, cap)
    vc, vs = P.empty_cache(B, Hkv, cap)
    iq.quantize_kv(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), rot, kc, ks, vc, vs)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return dict(q=torch.from_numpy(q).cuda(), kc=kc, ks=ks, vc=vc, vs=vs, rot=rot, lens=lens_t, params=params,
                lens_np=np.array(lens), q_np=q)


def _compare(c, label):
    ref = iq.decode_attention(c["q"], c["kc"], c["ks"], c["vc"], c["vs"], c["rot"], seq_lens=c["lens"])
    out = torch.full_like(ref, float("nan"))
    iq.decode_attention_noalloc(c["q"], c["kc"], c["ks"], c["vc"], c["vs"], c["rot"], seq_lens=c["lens"], out=out)
    torch.cuda.synchronize()
    print("%s: max |noalloc - workspace| = %g" % (label, float((out - ref).abs().max())), flush=True)
    assert torch.equal(out, ref), label
    return out


def test_noalloc_equals_workspace_call_twice_second_smaller():
    print("noalloc call 1: B=6, 32 query / 4 KV heads, cap 4096, ragged lengths", flush=True)
    big = _case(11, 6, 32, 4, 4096, [4096, 1, 0, 3000, 2048, 777])
    out1 = _compare(big, "call 1")
    # the first call against the oracle too (GPU codes fed to the oracle)
    b = 3
    n = int(big["lens_np"][b])
    ref = oracle.decode_attention(big["q_np"][b:b + 1].astype(np.float64),
                                  oracle.unpack(big["kc"][b:b + 1, :, :n].cpu().numpy()), big["ks"][b:b + 1, :, :n].cpu().numpy(),
                                  oracle.unpack(big["vc"][b:b + 1, :, :n].cpu().numpy()), big["vs"][b:b + 1, :, :n].cpu().numpy(),
                                  big["params"][b:b + 1], np.array([n]))
    P.check_output(out1[b:b + 1].cpu().numpy(), ref, what="noalloc vs oracle")
    print("noalloc call 2: B=2, 8 query / 2 KV heads, cap 640", flush=True)
    small = _case(12, 2, 8, 2, 640, [640, 129])
    _compare(small, "call 2")


def test_noalloc_refuses_sizes_beyond_its_scratch():
    # 20000 sequences of 8 query heads: 20000 partial rows per query head, about 83 MB of partials.
    # Validation refuses it before anything is launched; the buffers are never read.
    B, Hq, Hkv, cap = 20000, 8, 1, 256
    ws_need = iq.decode_workspace_bytes(B, Hq, Hkv, cap)
    assert ws_need > iq.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    kc = torch.zeros((B, Hkv, cap, 48), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Hkv, cap), dtype=torch.float32, device="cuda")
    rot = torch.zeros((B, Hkv, 32, 8), dtype=torch.float32, device="cuda")
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(iq.IQError) as e:
        iq.decode_attention_noalloc(q, kc, ks, kc, ks, rot, out=out)
    assert e.value.code == -3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0
