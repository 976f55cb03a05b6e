"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every entry point include/iq.h declares, argument validation returns the
documented error codes before anything is launched, and iq_make_rotation
reproduces the oracle's generator bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_space_decode_amd as iq
import oracle
from compressed_space_decode_amd import iq as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(iq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(["iq_last_error", "iq_make_rotation", "iq_quantize_kv",
                                  "iq_decode_workspace_bytes", "iq_decode_attention",
                                  "iq_decode_attention_append", "iq_decode_attention_multi",
                                  "iq_decode_attention_noalloc",
                                  "iq_quantize_kv_format", "iq_decode_attention_format",
                                  "iq_isotropy_workspace_bytes",
                                  "iq_isotropy_stats"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(iq.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(binding.SIGNATURES) == set(_declared())


def test_make_rotation_matches_oracle_bit_for_bit():
    for seed, n in [(0, 1), (1234567, 4), (2 ** 64 - 1, 3), (42, 192)]:
        got = iq.make_rotation(seed, n)
        want = oracle.make_rotation(seed, n)
        assert got.shape == (n, 32, 8)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_make_rotation_errors():
    lib = iq.lib()
    assert lib.iq_make_rotation(1, 0, ctypes.c_void_p(16)) == binding.IQ_EINVAL
    assert "n_heads" in binding.last_error()
    assert lib.iq_make_rotation(1, 2, None) == binding.IQ_EINVAL


FAKE = 1 << 20   # an aligned non-null address; validation fails before any use


def _quant(**kw):
    args = dict(k=FAKE, v=FAKE, dtype=1, n_seq=1, n_heads=1, n_tokens=4, ss=512, sh=512, st=128,
                rot=FAKE, rs=256, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, cap=4, off=0, hd=128, bits=3)
    args.update(kw)
    return iq.lib().iq_quantize_kv(args["k"], args["v"], args["dtype"], args["n_seq"], args["n_heads"],
                                   args["n_tokens"], args["ss"], args["sh"], args["st"], args["rot"], args["rs"],
                                   args["kc"], args["ks"], args["vc"], args["vs"], args["cap"], args["off"],
                                   args["hd"], args["bits"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(hd=64), binding.IQ_EUNSUPPORTED),
    (dict(bits=4), binding.IQ_EUNSUPPORTED),
    (dict(dtype=7), binding.IQ_EUNSUPPORTED),
    (dict(k=None, v=None), binding.IQ_EINVAL),
    (dict(kc=None), binding.IQ_EINVAL),
    (dict(rot=None), binding.IQ_EINVAL),
    (dict(n_seq=0), binding.IQ_EINVAL),
    (dict(n_heads=70000), binding.IQ_EINVAL),
    (dict(n_tokens=-1), binding.IQ_EINVAL),
    (dict(off=1), binding.IQ_EINVAL),            # 1 + 4 > cap
    (dict(st=-128), binding.IQ_EINVAL),
    (dict(st=100), binding.IQ_EINVAL),           # not a multiple of 16 bytes
    (dict(k=FAKE + 2), binding.IQ_EINVAL),       # misaligned input
    (dict(n_tokens=0), binding.IQ_OK),           # no-op, nothing launched
])
def test_quantize_validation(kw, code):
    assert _quant(**kw) == code
    if code != binding.IQ_OK:
        assert binding.last_error().startswith("iq_quantize_kv")


def _dec(**kw):
    args = dict(q=FAKE, qd=1, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, rot=FAKE, rs=0, lens=None, B=1, Hq=8, Hkv=2,
                cap=1000, sm=0.0, out=FAKE, ws=FAKE, wsb=1 << 30, hd=128, bits=3)
    args.update(kw)
    return iq.lib().iq_decode_attention(args["q"], args["qd"], args["kc"], args["ks"], args["vc"], args["vs"],
                                        args["rot"], args["rs"], args["lens"], args["B"], args["Hq"], args["Hkv"],
                                        args["cap"], args["sm"], args["out"], args["ws"], args["wsb"],
                                        args["hd"], args["bits"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(hd=96), binding.IQ_EUNSUPPORTED),
    (dict(bits=2), binding.IQ_EUNSUPPORTED),
    (dict(qd=3), binding.IQ_EUNSUPPORTED),
    (dict(Hq=6, Hkv=4), binding.IQ_EINVAL),
    (dict(B=0), binding.IQ_EINVAL),
    (dict(cap=0), binding.IQ_EINVAL),
    (dict(cap=83886017), binding.IQ_EINVAL),     # cache_cap * 48 must stay below 0xF0000000 - 64 * 48
    (dict(q=None), binding.IQ_EINVAL),
    (dict(vs=None), binding.IQ_EINVAL),
    (dict(rs=-1), binding.IQ_EINVAL),
    (dict(kc=FAKE + 1), binding.IQ_EINVAL),
    (dict(ws=None), binding.IQ_EWORKSPACE),
    (dict(wsb=16), binding.IQ_EWORKSPACE),
    (dict(ws=FAKE + 64), binding.IQ_EWORKSPACE),  # not 256-byte aligned
])
def test_decode_validation(kw, code):
    assert _dec(**kw) == code
    assert binding.last_error().startswith("iq_decode_attention")


def _app(**kw):
    args = dict(q=FAKE, qd=1, kn=FAKE, vn=FAKE, nd=1, nss=256, nsh=128, pos=FAKE, kc=FAKE, ks=FAKE, vc=FAKE,
                vs=FAKE, rot=FAKE, rs=0, B=1, Hq=8, Hkv=2, cap=1000, sm=0.0, out=FAKE, ws=FAKE, wsb=16,
                hd=128, bits=3)
    args.update(kw)
    return iq.lib().iq_decode_attention_append(
        args["q"], args["qd"], args["kn"], args["vn"], args["nd"], args["nss"], args["nsh"], args["pos"],
        args["kc"], args["ks"], args["vc"], args["vs"], args["rot"], args["rs"], args["B"], args["Hq"], args["Hkv"],
        args["cap"], args["sm"], args["out"], args["ws"], args["wsb"], args["hd"], args["bits"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(), binding.IQ_EWORKSPACE),             # everything valid but the 16-byte workspace
    (dict(hd=64), binding.IQ_EUNSUPPORTED),
    (dict(nd=7), binding.IQ_EUNSUPPORTED),
    (dict(qd=7), binding.IQ_EUNSUPPORTED),
    (dict(Hq=6, Hkv=4), binding.IQ_EINVAL),
    (dict(kn=None), binding.IQ_EINVAL),
    (dict(vn=None), binding.IQ_EINVAL),
    (dict(pos=None), binding.IQ_EINVAL),
    (dict(kn=FAKE + 8), binding.IQ_EINVAL),      # new vectors must be 16-byte aligned
    (dict(nsh=4), binding.IQ_EINVAL),            # 8 bytes of bf16: not a multiple of 16 bytes
    (dict(nss=-8), binding.IQ_EINVAL),
    (dict(pos=FAKE + 2), binding.IQ_EINVAL),
    (dict(cap=83886017), binding.IQ_EINVAL),
])
def test_decode_append_validation(kw, code):
    assert _app(**kw) == code
    assert binding.last_error().startswith("iq_decode_attention_append")


def test_workspace_bytes():
    n = iq.decode_workspace_bytes(1, 32, 4, 32768)
    assert n > 0
    # a plan head (256 bytes, then one int per sequence rounded up to 256 bytes), then partials:
    # (o' [128] + max + sum) floats per (work item, query head)
    assert (n - 512) % (130 * 4 * 32) == 0
    n16 = iq.decode_workspace_bytes(16, 32, 8, 32768)
    assert (n16 - 512) % (130 * 4 * 32) == 0
    n100 = iq.decode_workspace_bytes(100, 8, 8, 1000)
    assert (n100 - 256 - 512) % (130 * 4 * 8) == 0
    assert (n100 - 768) // (130 * 4 * 8) >= 100             # at least one work item per sequence
    assert iq.lib().iq_decode_workspace_bytes(1, 6, 4, 100) == binding.IQ_EINVAL
    assert iq.decode_workspace_bytes(16, 32, 8, 32768) >= iq.decode_workspace_bytes(1, 32, 8, 32768)
    assert iq.decode_workspace_bytes(1, 32, 4, 83886016) > 0          # the largest capacity
    assert iq.lib().iq_decode_workspace_bytes(1, 32, 4, 83886017) == binding.IQ_EINVAL


def _iso(**kw):
    args = dict(x=FAKE, dt=1, S=2, H=4, T=1000, ss=4 * 1000 * 128, sh=1000 * 128, st=128, tr=3, rot=FAKE, rs=1024,
                dense=None, ds=0, stats=FAKE, ws=FAKE, wsb=1 << 30)
    args.update(kw)
    return iq.lib().iq_isotropy_stats(args["x"], args["dt"], args["S"], args["H"], args["T"], args["ss"], args["sh"],
                                      args["st"], args["tr"], args["rot"], args["rs"], args["dense"], args["ds"],
                                      args["stats"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), binding.IQ_EUNSUPPORTED),
    (dict(tr=5), binding.IQ_EUNSUPPORTED),
    (dict(tr=-1), binding.IQ_EUNSUPPORTED),
    (dict(S=0), binding.IQ_EINVAL),
    (dict(H=70000), binding.IQ_EINVAL),
    (dict(T=-1), binding.IQ_EINVAL),
    (dict(stats=None), binding.IQ_EINVAL),
    (dict(stats=FAKE + 4), binding.IQ_EINVAL),       # doubles: 8-byte aligned
    (dict(x=None), binding.IQ_EINVAL),
    (dict(rot=None), binding.IQ_EINVAL),              # the method's transform needs the SO(4) params
    (dict(tr=2, rs=-1), binding.IQ_EINVAL),
    (dict(tr=4), binding.IQ_EINVAL),                  # dense transform without a matrix
    (dict(st=100), binding.IQ_EINVAL),                # not a multiple of 16 bytes
    (dict(x=FAKE + 8), binding.IQ_EINVAL),
    (dict(ws=None), binding.IQ_EWORKSPACE),
    (dict(wsb=1000), binding.IQ_EWORKSPACE),
    (dict(ws=FAKE + 128), binding.IQ_EWORKSPACE),
])
def test_isotropy_validation(kw, code):
    assert _iso(**kw) == code
    assert binding.last_error().startswith("iq_isotropy_stats")


def test_isotropy_workspace_bytes():
    # y_ref [128] plus (4 moments x 128 + 8 scalars) floats per 256 tokens, per (sequence, head)
    n = iq.isotropy_workspace_bytes(2, 3, 1000)
    assert n == 2 * 3 * (128 + 4 * (4 * 128 + 8)) * 4 + 256
    assert iq.isotropy_workspace_bytes(1, 1, 0) == 128 * 4 + 256
    assert iq.lib().iq_isotropy_workspace_bytes(0, 1, 10) == binding.IQ_EINVAL


def _multi(**kw):
    args = dict(q=FAKE, qd=1, Q=4, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, rot=FAKE, rs=0, lens=None, B=2, Hq=8, Hkv=2,
                cap=1000, sm=0.0, out=FAKE, ws=FAKE, wsb=16, hd=128, bits=3)
    args.update(kw)
    return iq.lib().iq_decode_attention_multi(
        args["q"], args["qd"], args["Q"], args["kc"], args["ks"], args["vc"], args["vs"], args["rot"], args["rs"],
        args["lens"], args["B"], args["Hq"], args["Hkv"], args["cap"], args["sm"], args["out"], args["ws"],
        args["wsb"], args["hd"], args["bits"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(), binding.IQ_EWORKSPACE),             # everything valid but the 16-byte workspace
    (dict(Q=0), binding.IQ_EINVAL),
    (dict(B=20000, Q=4), binding.IQ_EINVAL),      # batch * n_q_tokens > 65535
    (dict(qd=5), binding.IQ_EUNSUPPORTED),
    (dict(hd=64), binding.IQ_EUNSUPPORTED),
    (dict(q=None), binding.IQ_EINVAL),
    (dict(Hq=6, Hkv=4), binding.IQ_EINVAL),
    (dict(q=FAKE + 4), binding.IQ_EINVAL),
])
def test_decode_multi_validation(kw, code):
    assert _multi(**kw) == code
    assert binding.last_error().startswith("iq_decode_attention_multi")


def test_decode_multi_workspace_is_that_of_batch_times_tokens():
    need = iq.decode_workspace_bytes(2 * 4, 8, 2, 1000)
    assert _multi(wsb=need - 1) == binding.IQ_EWORKSPACE


def _qfmt(fmt, **kw):
    args = dict(k=FAKE, v=FAKE, dtype=1, n_seq=1, n_heads=1, n_tokens=4, ss=512, sh=512, st=128,
                rot=FAKE, rs=256, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, cap=4, off=0, hd=128)
    args.update(kw)
    return iq.lib().iq_quantize_kv_format(args["k"], args["v"], args["dtype"], args["n_seq"], args["n_heads"],
                                          args["n_tokens"], args["ss"], args["sh"], args["st"], args["rot"],
                                          args["rs"], args["kc"], args["ks"], args["vc"], args["vs"], args["cap"],
                                          args["off"], args["hd"], fmt, None)


def test_format_entry_points_validate():
    assert _qfmt(7) == binding.IQ_EUNSUPPORTED and "format" in binding.last_error()
    assert _qfmt(-1) == binding.IQ_EUNSUPPORTED
    assert _qfmt(1, hd=64) == binding.IQ_EUNSUPPORTED
    assert _qfmt(2, kc=FAKE + 4) == binding.IQ_EINVAL            # 4-bit records: 8-byte aligned codes
    assert "8-byte" in binding.last_error()
    assert _qfmt(3, n_tokens=0) == binding.IQ_OK                  # nothing to do
    assert _qfmt(1, off=1) == binding.IQ_EINVAL
    lib = iq.lib()
    rc = lib.iq_decode_attention_format(FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, 1, 8, 2, 1000, 0.0, FAKE,
                                        FAKE, 16, 128, 9, None)
    assert rc == binding.IQ_EUNSUPPORTED and binding.last_error().startswith("iq_decode_attention_format")
    rc = lib.iq_decode_attention_format(FAKE, 1, FAKE + 4, FAKE, FAKE, FAKE, FAKE, 0, None, 1, 8, 2, 1000, 0.0, FAKE,
                                        FAKE, 1 << 30, 128, 2, None)
    assert rc == binding.IQ_EINVAL
    rc = lib.iq_decode_attention_format(FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, 1, 8, 2, 1000, 0.0, FAKE,
                                        FAKE, 16, 128, 1, None)
    assert rc == binding.IQ_EWORKSPACE
    # the asymmetric format's (s, m) scale pairs must be 8-byte aligned, in both entry points
    assert _qfmt(4, ks=FAKE + 4) == binding.IQ_EINVAL and "(s, m)" in binding.last_error()
    rc = lib.iq_decode_attention_format(FAKE, 1, FAKE, FAKE, FAKE, FAKE + 4, FAKE, 0, None, 1, 8, 2, 1000, 0.0, FAKE,
                                        FAKE, 1 << 30, 128, 4, None)
    assert rc == binding.IQ_EINVAL and "(s, m)" in binding.last_error()
    assert _qfmt(5) == binding.IQ_EUNSUPPORTED                    # past the last format


def test_probe_library_exports_and_validates():
    # the measurement library beside libiq.so: its two symbols (default and non-temporal loads),
    # and argument checks before any launch
    probe = binding.probe_lib()
    for name in ("iq_probe_stream_read", "iq_probe_stream_read_nt"):
        fn = getattr(probe, name)
        assert fn(None, 1024, 64, FAKE, None) == -1
        assert fn(FAKE, 1000, 64, FAKE, None) == -1       # not a multiple of 16
        assert fn(FAKE + 4, 1024, 64, FAKE, None) == -1   # misaligned
        assert fn(FAKE, 1024, 0, FAKE, None) == -1
        assert fn(FAKE, 1024, 70000, FAKE, None) == -1
        assert fn(FAKE, 1024, 64, None, None) == -1
