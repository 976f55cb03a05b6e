"""Parity helpers shared by the GPU tests: run the HIP path through the C ABI
binding and compare with the CPU oracle to the stated tolerances.

Tolerances (stated once, used everywhere):
  * packed codes: bit-exact, except that a fraction <= 1e-4 of the codes may
    differ by exactly one level, and only where the oracle's fp64 rotated
    value lies within 1e-6 * max|x'| of a decision threshold (fp32 rounding
    in the kernel can land on either side of such a threshold);
  * scales: within 1e-6 relative;
  * attention output: max abs error <= 2e-3 (fp32 accumulation).
"""
import numpy as np

import oracle

FLIP_FRACTION = 1e-4
FLIP_DIST = 3.5e-6          # 1e-6 * absmax, in units of the step s = absmax / 3.5
SCALE_RTOL = 1e-6
OUT_ATOL = 2e-3


def torch_input(x, dtype, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def empty_cache(n_seq, n_heads, cap, device="cuda", poison=False):
    import torch
    codes = torch.zeros((n_seq, n_heads, cap, 48), dtype=torch.uint8, device=device)
    scales = torch.zeros((n_seq, n_heads, cap), dtype=torch.float32, device=device)
    if poison:
        codes.fill_(0xFF)
        scales.fill_(1e30)
    return codes, scales


def check_quantize(x64, params, records, scales, what=""):
    """x64 [N][128] fp64 inputs of one (sequence, head); records uint8 [N][48] and
    scales float32 [N] from the GPU.  Every differing code must be a one-level
    flip next to a threshold; the caller bounds the total flip fraction.
    Returns (n_flips, worst_flip_distance)."""
    codes_o, scales_o, xr, s = oracle.quantize(x64, params)
    codes_g = oracle.unpack(records)
    mism = codes_g != codes_o
    n = int(mism.sum())
    worst = 0.0
    if n:
        rows, cols = np.nonzero(mism)
        assert np.all(np.abs(codes_g[mism].astype(int) - codes_o[mism].astype(int)) == 1), what
        u = xr[rows, cols] / s[rows] + 4.0
        k = np.rint(u)
        dist = np.abs(u - k)
        worst = float(dist.max())
        assert np.all((k >= 1) & (k <= 7)), what
        assert worst <= FLIP_DIST, "%s: code flip %.3g from a threshold" % (what, worst)
        ok_rows = ~np.any(mism, axis=1)
    else:
        ok_rows = np.ones(len(records), dtype=bool)
    np.testing.assert_array_equal(records[ok_rows], oracle.pack(codes_o[ok_rows]), err_msg=what)
    np.testing.assert_allclose(scales, scales_o.astype(np.float64), rtol=SCALE_RTOL, atol=0, err_msg=what)
    return n, worst


def check_output(out_gpu, out_oracle, what=""):
    err = float(np.max(np.abs(np.asarray(out_gpu, np.float64) - out_oracle))) if out_oracle.size else 0.0
    assert err <= OUT_ATOL, "%s: max abs error %.3g" % (what, err)
    return err
