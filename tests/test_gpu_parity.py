"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
five synthetic workloads, at their full sizes.  Quantize: every vector (tiny,
gqa8k, long32k) or sampled (sequence, head) pairs (ragged, prefill).  Decode:
every output row, with the oracle fed the codes the GPU produced.  The
benchmark's timed step (48 long32k layers, fused append) at its full size and
launch configuration: sampled layers, every head.

Tolerances are stated in tests/_parity.py.
"""
import numpy as np
import pytest
import torch

import _parity as P
import compressed_space_decode_amd as iq
import oracle
from compressed_space_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _run_workload(name, batch=None, tokens=None, poison_tail=False):
    """Generate a decode workload, quantize K/V on the GPU, return host copies."""
    _log("workload %s batch=%s tokens=%s" % (name, batch, tokens))
    w = W.decode_workload(name, batch=batch, tokens=tokens)
    B, Hkv, T = w["k"].shape[:3]
    dev = "cuda"
    kt = P.torch_input(w["k"], w["dtype"], dev)
    vt = P.torch_input(w["v"], w["dtype"], dev)
    rot = torch.from_numpy(w["params"]).to(dev)
    kc, ks = P.empty_cache(B, Hkv, T, dev)
    vc, vs = P.empty_cache(B, Hkv, T, dev)
    iq.quantize_kv(kt, vt, rot, kc, ks, vc, vs)
    torch.cuda.synchronize()
    del kt, vt
    if poison_tail:
        for b in range(B):
            n = int(w["seq_lens"][b])
            kc[b, :, n:] = 0xFF
            vc[b, :, n:] = 0xFF
            ks[b, :, n:] = 1e30
            vs[b, :, n:] = 1e30
    q = P.torch_input(w["q"], w["dtype"], dev)
    lens = torch.from_numpy(w["seq_lens"]).to(dev)
    out = iq.decode_attention(q, kc, ks, vc, vs, rot, seq_lens=lens)
    torch.cuda.synchronize()
    w["gpu"] = dict(kc=kc.cpu().numpy(), ks=ks.cpu().numpy(), vc=vc.cpu().numpy(), vs=vs.cpu().numpy(),
                    out=out.cpu().numpy())
    return w


def _check_quantize_pairs(w, pairs, token_sel=None):
    """Check quantization of the given (b, h) pairs (all tokens, or token_sel)."""
    flips, total = 0, 0
    worst = 0.0
    for b, h in pairs:
        n_valid = int(w["seq_lens"][b])     # positions past the length may be poisoned
        for side in ("k", "v"):
            x = w[side][b, h]
            idx = np.arange(n_valid) if token_sel is None else token_sel[token_sel < n_valid]
            x64 = W.to_f64(x[idx], w["dtype"])
            rec = w["gpu"][side[0] + "c"][b, h][idx]
            sc = w["gpu"][side[0] + "s"][b, h][idx]
            n, dist = P.check_quantize(x64, w["params"][b, h], rec, sc, what="%s %s b=%d h=%d" % (w["workload"], side, b, h))
            flips += n
            worst = max(worst, dist)
            total += x64.size
    assert flips <= P.FLIP_FRACTION * total, "%d threshold flips in %d codes" % (flips, total)
    _log("  quantize: %d codes, %d threshold flips (worst distance %.2g)" % (total, flips, worst))


def _check_decode(w, rows=None):
    g = w["gpu"]
    B = w["q"].shape[0]
    q64 = W.to_f64(w["q"], w["dtype"])
    bs = range(B) if rows is None else rows
    errs = []
    for b in bs:
        n = int(w["seq_lens"][b])
        kcodes = oracle.unpack(g["kc"][b:b + 1, :, :n])
        vcodes = oracle.unpack(g["vc"][b:b + 1, :, :n])
        ref = oracle.decode_attention(q64[b:b + 1], kcodes, g["ks"][b:b + 1, :, :n], vcodes, g["vs"][b:b + 1, :, :n],
                                      w["params"][b:b + 1], np.array([n]))
        errs.append(P.check_output(g["out"][b:b + 1], ref, what="%s b=%d len=%d" % (w["workload"], b, n)))
    _log("  decode: max abs error %.3g over %d sequences" % (max(errs), len(errs)))
    return max(errs)


@pytest.fixture(scope="module")
def tiny():
    return _run_workload("tiny")


@pytest.fixture(scope="module")
def gqa8k():
    return _run_workload("gqa8k")


@pytest.fixture(scope="module")
def long32k():
    return _run_workload("long32k")


@pytest.fixture(scope="module")
def ragged():
    return _run_workload("ragged", poison_tail=True)


def test_tiny_quantize(tiny):
    _check_quantize_pairs(tiny, [(0, h) for h in range(4)])


def test_tiny_decode(tiny):
    _check_decode(tiny)


def test_gqa8k_quantize(gqa8k):
    _check_quantize_pairs(gqa8k, [(0, h) for h in range(4)])


def test_gqa8k_decode(gqa8k):
    _check_decode(gqa8k)


def test_long32k_quantize(long32k):
    _check_quantize_pairs(long32k, [(0, h) for h in range(4)])


def test_long32k_decode(long32k):
    _check_decode(long32k)


def test_long32k_planted_key_retrieval(long32k):
    # Property, not parity: the stand-in for the Abstract's retrieval at 32K context.  For each KV
    # head, is the planted position the argmax of the exact fp64 scores q.k (unquantized K) and of
    # the 3-bit compressed-space scores (R q).k_hat on the GPU's codes, for the query head the key
    # was planted for (its KV group's first head)?  Both results are logged per head.  The 3-bit
    # scores must keep every head the exact scores retrieve.  On this seeded workload the exact
    # scores themselves miss KV head 0: another key's channel-scaled score beats the planted key's
    # before any quantization, so that head cannot count against the quantizer.
    w, g = long32k, long32k["gpu"]
    p = int(w["planted_pos"][0])
    q64 = W.to_f64(w["q"], w["dtype"])
    G = w["n_q_heads"] // w["n_kv_heads"]
    exact, packed = [], []
    for h in range(w["n_kv_heads"]):
        qh = q64[0, h * G]
        ze = W.to_f64(w["k"][0, h], w["dtype"]) @ qh
        R = oracle.rotation_matrix(w["params"][0, h])
        z3 = oracle.dequantize_rotated(oracle.unpack(g["kc"][0, h]), g["ks"][0, h]) @ (R @ qh)
        exact.append(int(np.argmax(ze)))
        packed.append(int(np.argmax(z3)))
        _log("  KV head %d: planted %d; exact argmax %d (%s), 3-bit argmax %d (%s)" %
             (h, p, exact[-1], "hit" if exact[-1] == p else "miss", packed[-1], "hit" if packed[-1] == p else "miss"))
    hits_exact = [e == p for e in exact]
    hits_packed = [c == p for c in packed]
    _log("  planted key retrieved: exact %d of %d, 3-bit %d of %d" %
         (sum(hits_exact), len(exact), sum(hits_packed), len(packed)))
    assert all(hp for he, hp in zip(hits_exact, hits_packed) if he), "3-bit lost a head the exact scores retrieve"
    assert hits_exact == [False, True, True, True], "the seeded workload's exact retrieval changed"


def test_ragged_quantize_sampled(ragged):
    rng = np.random.default_rng(0)
    pairs = [(0, 0), (15, 7)] + [(int(rng.integers(16)), int(rng.integers(8))) for _ in range(2)]
    _check_quantize_pairs(ragged, pairs[:2])
    sel = np.sort(rng.choice(32768, size=2048, replace=False))
    _check_quantize_pairs(ragged, pairs[2:], token_sel=sel)


def test_ragged_decode_poisoned_padding(ragged):
    assert ragged["seq_lens"].min() >= 1024
    _check_decode(ragged)


def test_prefill_full_size_sampled():
    layers, H, T = W.PREFILL_SHAPE
    _log("prefill: generating %d layers" % layers)
    data = W.prefill_layers(range(layers))
    k = torch.empty((layers, H, T, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    params = np.stack([d[2] for d in data])
    for l, (kk, vv, _) in enumerate(data):
        k[l] = P.torch_input(kk, "bf16")
        v[l] = P.torch_input(vv, "bf16")
    rot = torch.from_numpy(params).cuda()
    kc, ks = P.empty_cache(layers, H, T)
    vc, vs = P.empty_cache(layers, H, T)
    iq.quantize_kv(k, v, rot, kc, ks, vc, vs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    sel = np.sort(rng.choice(T, size=1024, replace=False))
    sel = np.unique(np.concatenate([sel, [0, T - 1]]))
    flips, total = 0, 0
    for l in (0, 23, 47):
        for h in range(H):
            for side, c, s in (("k", kc, ks), ("v", vc, vs)):
                x = data[l][0 if side == "k" else 1][h][sel]
                n, _ = P.check_quantize(W.to_f64(x, "bf16"), params[l, h], c[l, h, sel].cpu().numpy(),
                                        s[l, h, sel].cpu().numpy(), what="prefill l=%d h=%d %s" % (l, h, side))
                flips += n
                total += x.size
    assert flips <= P.FLIP_FRACTION * total
    _log("  prefill quantize: %d sampled codes, %d threshold flips" % (total, flips))


def test_long32k_48_layer_append_step_sampled():
    # The benchmark's timed step at its full size and launch configuration: 48 layers stacked as
    # batch entries (32 query / 4 KV heads, 32768 cached tokens each) and one
    # iq_decode_attention_append launch that writes the new token at position 32767 and attends over
    # all 32768.  Every layer's appended records must equal iq_quantize_kv's; the outputs of three
    # layers (every head) are checked against the oracle on the GPU's codes.
    L = 48
    _log("long32k x%d append step" % L)
    w = W.decode_workload("long32k", batch=L)
    B, Hkv, T = w["k"].shape[:3]
    kt = P.torch_input(w["k"], w["dtype"])
    vt = P.torch_input(w["v"], w["dtype"])
    rot = torch.from_numpy(w["params"]).cuda()
    kc, ks = P.empty_cache(B, Hkv, T)
    vc, vs = P.empty_cache(B, Hkv, T)
    iq.quantize_kv(kt[:, :, :T - 1], vt[:, :, :T - 1], rot, kc, ks, vc, vs)   # the prefilled context
    kc[:, :, T - 1] = 0xAB                                                      # the slot the step writes
    vc[:, :, T - 1] = 0xAB
    q = P.torch_input(w["q"], w["dtype"])
    positions = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(iq.decode_workspace_bytes(B, w["q"].shape[1], Hkv, T), dtype=torch.uint8, device="cuda")
    out = iq.decode_attention_append(q, kt[:, :, T - 1], vt[:, :, T - 1], positions, kc, ks, vc, vs, rot, workspace=ws)
    # the same records by the separate quantize call
    kc2, ks2 = P.empty_cache(B, Hkv, 1)
    vc2, vs2 = P.empty_cache(B, Hkv, 1)
    iq.quantize_kv(kt[:, :, T - 1:], vt[:, :, T - 1:], rot, kc2, ks2, vc2, vs2)
    torch.cuda.synchronize()
    assert torch.equal(kc[:, :, T - 1], kc2[:, :, 0]) and torch.equal(vc[:, :, T - 1], vc2[:, :, 0])
    assert torch.equal(ks[:, :, T - 1], ks2[:, :, 0]) and torch.equal(vs[:, :, T - 1], vs2[:, :, 0])
    del kt, vt, kc2, vc2, ks2, vs2
    g = dict(kc=kc.cpu().numpy(), ks=ks.cpu().numpy(), vc=vc.cpu().numpy(), vs=vs.cpu().numpy(),
             out=out.cpu().numpy())
    w["gpu"] = g
    w["seq_lens"] = np.full(B, T, dtype=np.int32)
    _check_decode(w, rows=(0, 23, 47))
    # the appended records of the sampled layers against the oracle's quantization of the new token
    flips = 0
    for b in (0, 23, 47):
        for h in range(Hkv):
            for side, c, s in (("k", g["kc"], g["ks"]), ("v", g["vc"], g["vs"])):
                x64 = W.to_f64(w[side][b, h, T - 1:T], w["dtype"])
                n, _ = P.check_quantize(x64, w["params"][b, h], c[b, h, T - 1:T], s[b, h, T - 1:T],
                                        what="appended %s b=%d h=%d" % (side, b, h))
                flips += n
    assert flips <= 1
