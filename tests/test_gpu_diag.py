"""GPU parity of the isotropy diagnostics (iq_isotropy_stats) against the
oracle (oracle/diagnostics.py), through the C ABI.

Every transform, fp32 and bf16 inputs, token counts that span several
256-token partials with a ragged tail, strided inputs, shared parameters, and
the degenerate cases (no tokens, a coordinate that never changes, zero
vectors).  Tolerances: the statistics are ratios of fp32 sums that the
kernels add in fp64, compared with fp64 values: relative 1e-4 (absolute 1e-9
for values near zero); the token count is exact.
"""
import numpy as np
import pytest
import torch

import compressed_space_decode_amd as iq
from compressed_space_decode_amd import workloads as W
from oracle import diagnostics as Dg

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-9


def _params(rng, *lead):
    g = rng.standard_normal(lead + (32, 2, 4))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    return g.reshape(lead + (32, 8)).astype(np.float32)


def _orthogonal(rng, *lead):
    a = rng.standard_normal(lead + (128, 128))
    q, r = np.linalg.qr(a)
    return (q * np.sign(np.diagonal(r, axis1=-2, axis2=-1))[..., None, :]).astype(np.float32)


def _inputs(rng, S, H, T):
    """Heavy tails (Student-t 3) plus a few large channels per head: far from isotropic."""
    x = rng.standard_t(3, size=(S, H, T, 128)).astype(np.float32)
    for s in range(S):
        for h in range(H):
            x[s, h, :, rng.choice(128, size=3, replace=False)] *= 12.0
    return x


def _compare(got, x64, mode, params, dense, what):
    S, H = x64.shape[:2]
    for s in range(S):
        for h in range(H):
            want = Dg.isotropy_stats(x64[s, h], mode, None if params is None else params[s, h],
                                     None if dense is None else dense[s, h])
            g = got[s, h]
            assert g[Dg.I_COUNT] == want[Dg.I_COUNT], what
            np.testing.assert_allclose(g, want, rtol=RTOL, atol=ATOL, err_msg="%s s=%d h=%d" % (what, s, h))


@pytest.mark.parametrize("mode", ["none", "wht", "so4", "wht_so4", "dense"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_isotropy_stats_match_oracle(mode, dtype):
    rng = np.random.default_rng(100 + Dg.TRANSFORMS.index(mode) + (10 if dtype == "bf16" else 0))
    S, H, T = 2, 3, 777                              # three full 256-token partials and a tail of 9
    x = _inputs(rng, S, H, T)
    xin = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    params = _params(rng, S, H)
    dense = _orthogonal(rng, S, H)
    xt = torch.from_numpy(np.ascontiguousarray(xin).view(np.int16)).view(torch.bfloat16).cuda() \
        if dtype == "bf16" else torch.from_numpy(x).cuda()
    got = iq.isotropy_stats(xt, mode, rot=torch.from_numpy(params).cuda(), dense=torch.from_numpy(dense).cuda())
    torch.cuda.synchronize()
    _compare(got.cpu().numpy(), W.to_f64(xin, dtype), mode, params, dense, "%s %s" % (mode, dtype))


def test_isotropy_strided_input_shared_parameters_and_permutation():
    rng = np.random.default_rng(120)
    big = _inputs(rng, 2, 2, 300)
    big = np.concatenate([big, big[..., :64]], axis=-1)             # [2][2][300][192]
    x = torch.from_numpy(big).cuda()[:, :, 20:280, 32:160]           # strides (115200, 57600, 192, 1)
    x64 = big[:, :, 20:280, 32:160].astype(np.float64)
    params = _params(rng, 2)
    got = iq.isotropy_stats(x, "wht_so4", rot=torch.from_numpy(params).cuda(), shared=True)
    _compare(got.cpu().numpy(), x64, "wht_so4", np.broadcast_to(params, (2, 2, 32, 8)), None, "strided, shared")
    perm = rng.permutation(128)
    P = np.zeros((2, 128, 128), dtype=np.float32)
    P[:, np.arange(128), perm] = 1.0
    got = iq.isotropy_stats(x, "dense", dense=torch.from_numpy(P).cuda(), shared=True)
    _compare(got.cpu().numpy(), x64, "dense", None, np.broadcast_to(P, (2, 2, 128, 128)), "permutation")


def test_isotropy_dense_outside_fp16_range():
    # the dense transform splits each vector into fp16 parts after scaling it by a power of two:
    # values far above fp16's largest (6.5e4) and far below its normal range (6e-5) give the same
    # statistics as the oracle; zero vectors stay zero
    rng = np.random.default_rng(123)
    x = _inputs(rng, 1, 2, 300)
    x[0, 0] *= np.float32(3e6)
    x[0, 1] *= np.float32(2e-9)
    x[0, 1, 50:60] = 0.0
    dense = _orthogonal(rng, 1, 2)
    got = iq.isotropy_stats(torch.from_numpy(x).cuda(), "dense", dense=torch.from_numpy(dense).cuda())
    _compare(got.cpu().numpy(), x.astype(np.float64), "dense", None, dense, "dense, wide range")


def test_isotropy_degenerate_inputs():
    rng = np.random.default_rng(121)
    T = 300
    x = rng.standard_normal((1, 3, T, 128)).astype(np.float32)
    x[0, 0, :, 7] = 3.25                              # a coordinate that never changes
    x[0, 1, 100:140] = 0.0                            # zero vectors among others
    x[0, 2] = 0.0                                     # a head with only zero vectors
    got = iq.isotropy_stats(torch.from_numpy(x).cuda(), "none").cpu().numpy()
    _compare(got, x.astype(np.float64), "none", None, None, "degenerate")
    assert got[0, 0, 7] == 0.0 and got[0, 0, 128 + 7] == 0.0
    assert np.all(got[0, 2, :259] == 0.0) and got[0, 2, Dg.I_COUNT] == T
    empty = iq.isotropy_stats(torch.zeros((1, 2, 0, 128), device="cuda"), "wht")
    assert torch.all(empty == 0)


def test_isotropy_workspace_reused_and_dirty():
    rng = np.random.default_rng(122)
    ws = torch.full((iq.isotropy_workspace_bytes(1, 2, 600),), 0x7F, dtype=torch.uint8, device="cuda")
    for T in (600, 257, 1):
        x = _inputs(rng, 1, 2, T)
        got = iq.isotropy_stats(torch.from_numpy(x).cuda(), "wht", workspace=ws).cpu().numpy()
        _compare(got, x.astype(np.float64), "wht", None, None, "reuse T=%d" % T)
