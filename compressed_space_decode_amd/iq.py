"""Thin Python binding of libiq (ctypes).  Argument marshalling only: every
step of the method runs in the HIP kernels behind the C ABI (include/iq.h).

PyTorch is used for device memory and the current HIP stream.  There is no
fallback: if libiq.so is missing or fails to load, importing the functions
raises.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libiq.so")

IQ_OK, IQ_EINVAL, IQ_EUNSUPPORTED, IQ_EWORKSPACE, IQ_EHIP = 0, -1, -2, -3, -4
IQ_F32, IQ_BF16 = 0, 1
HEAD_DIM, BITS, RECORD_BYTES, ROT_PARAMS = 128, 3, 48, 256
TRANSFORMS = {"none": 0, "wht": 1, "so4": 2, "wht_so4": 3, "dense": 4}   # IQ_T_*
FORMATS = {"u3": 0, "u2": 1, "u4": 2, "lm3": 3, "a3": 4}                 # IQ_FMT_*
FORMAT_BITS = {"u3": 3, "u2": 2, "u4": 4, "lm3": 3, "a3": 3}


def scale_shape(lead, fmt):
    """Shape of a scales array: one fp32 per vector, or the (s, m) pair of the asymmetric format."""
    return tuple(lead) + ((2,) if fmt == "a3" else ())
N_STATS = 260

# (name, restype, argtypes) of every entry point declared in include/iq.h
_P = ctypes.c_void_p
_I32, _I64, _U64, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
SIGNATURES = {
    "iq_last_error": (ctypes.c_char_p, []),
    "iq_make_rotation": (ctypes.c_int, [_U64, _I32, _P]),
    "iq_quantize_kv": (ctypes.c_int, [_P, _P, _I32, _I64, _I32, _I64, _I64, _I64, _I64, _P, _I64,
                                      _P, _P, _P, _P, _I64, _I64, _I32, _I32, _P]),
    "iq_decode_workspace_bytes": (_I64, [_I32, _I32, _I32, _I64]),
    "iq_decode_attention": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                           _I64, _F, _P, _P, _I64, _I32, _I32, _P]),
    "iq_decode_attention_append": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P,
                                                  _I64, _I32, _I32, _I32, _I64, _F, _P, _P, _I64, _I32, _I32,
                                                  _P]),
    "iq_decode_attention_multi": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                                 _I64, _F, _P, _P, _I64, _I32, _I32, _P]),
    "iq_decode_attention_noalloc": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                                   _I64, _F, _P, _I32, _I32, _P]),
    "iq_quantize_kv_format": (ctypes.c_int, [_P, _P, _I32, _I64, _I32, _I64, _I64, _I64, _I64, _P, _I64,
                                             _P, _P, _P, _P, _I64, _I64, _I32, _I32, _P]),
    "iq_decode_attention_format": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                                  _I64, _F, _P, _P, _I64, _I32, _I32, _P]),
    "iq_isotropy_workspace_bytes": (_I64, [_I64, _I32, _I64]),
    "iq_isotropy_stats": (ctypes.c_int, [_P, _I32, _I64, _I32, _I64, _I64, _I64, _I64, _I32, _P, _I64, _P, _I64,
                                         _P, _P, _I64, _P]),
}


class IQError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libiq error %d: %s" % (code, msg))
        self.code = code


_lib = None


def lib():
    """Load libiq.so once (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libiq.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(rc):
    if rc != IQ_OK:
        raise IQError(rc, lib().iq_last_error().decode())


def last_error():
    return lib().iq_last_error().decode()


# ----------------------------------------------------------------------------
def make_rotation(seed, n_heads):
    """float32 numpy [n_heads][32][8] rotation parameters (host, seeded)."""
    out = np.zeros((int(n_heads), 32, 8), dtype=np.float32)
    _check(lib().iq_make_rotation(int(seed) & ((1 << 64) - 1), int(n_heads), out.ctypes.data))
    return out


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return IQ_F32
    if t.dtype == torch.bfloat16:
        return IQ_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def quantize_kv(k, v, rot, k_codes, k_scales, v_codes, v_scales, tok_offset=0, shared_rot=False, fmt="u3"):
    """Quantize K and/or V [n_seq][n_heads][n_tokens][128] (cuda, f32/bf16, last dim
    contiguous) into the cache (codes uint8 [n_seq][n_heads][cap][16 * bits], scales float32
    [n_seq][n_heads][cap]).  ``rot`` is float32 [n_seq][n_heads][32][8] on the device
    (or [n_heads][32][8] with shared_rot=True).  Either k or v may be None.  ``fmt`` is a
    record format of FORMATS ("u3": the pages' 3-bit codes, iq_quantize_kv)."""
    ref = k if k is not None else v
    n_seq, n_heads, n_tokens, d = ref.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    for t in (k, v):
        if t is not None and (t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype):
            raise ValueError("k and v must share shape, strides and dtype")
        if t is not None and t.stride(3) != 1:
            raise ValueError("coordinates must be contiguous")
    cache = k_codes if k is not None else v_codes
    cap = cache.shape[2]
    for c, sc, t in ((k_codes, k_scales, k), (v_codes, v_scales, v)):
        if t is None:
            continue
        if (tuple(c.shape) != (n_seq, n_heads, cap, 16 * FORMAT_BITS[fmt])
                or tuple(sc.shape) != scale_shape((n_seq, n_heads, cap), fmt)
                or not c.is_contiguous() or not sc.is_contiguous()):
            raise ValueError("cache must be contiguous codes [n_seq][n_heads][cap][%d] and scales %s"
                             % (16 * FORMAT_BITS[fmt], "[n_seq][n_heads][cap]" + ("[2]" if fmt == "a3" else "")))
    want_rot = (n_heads if shared_rot else n_seq * n_heads) * ROT_PARAMS
    if rot.numel() != want_rot or not rot.is_contiguous():
        raise ValueError("rot must be a contiguous float32 tensor of %d values" % want_rot)
    rot_stride = 0 if shared_rot else n_heads * ROT_PARAMS
    args = (k.data_ptr() if k is not None else None, v.data_ptr() if v is not None else None,
            _dtype_code(ref), n_seq, n_heads, n_tokens,
            ref.stride(0), ref.stride(1), ref.stride(2),
            rot.data_ptr(), rot_stride,
            k_codes.data_ptr() if k is not None else None, k_scales.data_ptr() if k is not None else None,
            v_codes.data_ptr() if v is not None else None, v_scales.data_ptr() if v is not None else None,
            cap, int(tok_offset), HEAD_DIM)
    if fmt == "u3":
        rc = lib().iq_quantize_kv(*args, BITS, _stream(ref))
    else:
        rc = lib().iq_quantize_kv_format(*args, FORMATS[fmt], _stream(ref))
    _check(rc)


def decode_workspace_bytes(batch, n_q_heads, n_kv_heads, cache_cap):
    n = lib().iq_decode_workspace_bytes(int(batch), int(n_q_heads), int(n_kv_heads), int(cache_cap))
    if n < 0:
        raise IQError(int(n), last_error())
    return int(n)


def decode_attention(q, k_codes, k_scales, v_codes, v_scales, rot, seq_lens=None, sm_scale=0.0,
                     out=None, workspace=None, shared_rot=False, fmt="u3"):
    """One decode step on the packed cache.  q [B][Hq][128] (cuda f32/bf16, contiguous);
    caches [B][Hkv][cap][48] / [B][Hkv][cap]; rot float32 [B][Hkv][32][8] (or [Hkv][32][8]
    with shared_rot=True); seq_lens int32 [B] on the device or None.  Returns out
    float32 [B][Hq][128]."""
    import torch
    B, Hq, d = q.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    if d != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [B][Hq][128]")
    for t in (k_codes, k_scales, v_codes, v_scales, rot):
        if not t.is_contiguous():
            raise ValueError("cache and rotation tensors must be contiguous")
    for c, sc in ((k_codes, k_scales), (v_codes, v_scales)):
        if tuple(c.shape) != (B, Hkv, cap, 16 * FORMAT_BITS[fmt]) or tuple(sc.shape) != scale_shape((B, Hkv, cap), fmt):
            raise ValueError("caches must be [B][Hkv][cap][%d] codes and %s scales"
                             % (16 * FORMAT_BITS[fmt], "[B][Hkv][cap]" + ("[2]" if fmt == "a3" else "")))
    if rot.numel() != (Hkv if shared_rot else B * Hkv) * ROT_PARAMS:
        raise ValueError("rot has the wrong number of values")
    if seq_lens is not None and seq_lens.numel() != B:
        raise ValueError("seq_lens must hold one length per sequence")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, Hq, Hkv, cap)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous()):
        raise ValueError("seq_lens must be a contiguous int32 tensor")
    args = (q.data_ptr(), _dtype_code(q), k_codes.data_ptr(), k_scales.data_ptr(),
            v_codes.data_ptr(), v_scales.data_ptr(), rot.data_ptr(),
            0 if shared_rot else Hkv * ROT_PARAMS,
            seq_lens.data_ptr() if seq_lens is not None else None,
            B, Hq, Hkv, cap, float(sm_scale), out.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), HEAD_DIM)
    if fmt == "u3":
        rc = lib().iq_decode_attention(*args, BITS, _stream(q))
    else:
        rc = lib().iq_decode_attention_format(*args, FORMATS[fmt], _stream(q))
    _check(rc)
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20   # IQ_NOALLOC_SCRATCH_BYTES


def decode_attention_noalloc(q, k_codes, k_scales, v_codes, v_scales, rot, seq_lens=None, sm_scale=0.0,
                             out=None, shared_rot=False):
    """decode_attention without a workspace (iq_decode_attention_noalloc): the library's own
    per-device scratch holds the split-K partials.  Same arguments and result; `out` must be given
    when no allocation may happen (else it is allocated here)."""
    import torch
    B, Hq, d = q.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    if d != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [B][Hq][128]")
    for t in (k_codes, k_scales, v_codes, v_scales, rot):
        if not t.is_contiguous():
            raise ValueError("cache and rotation tensors must be contiguous")
    for c, sc in ((k_codes, k_scales), (v_codes, v_scales)):
        if tuple(c.shape) != (B, Hkv, cap, RECORD_BYTES) or tuple(sc.shape) != (B, Hkv, cap):
            raise ValueError("caches must be [B][Hkv][cap][48] codes and [B][Hkv][cap] scales")
    if rot.numel() != (Hkv if shared_rot else B * Hkv) * ROT_PARAMS:
        raise ValueError("rot has the wrong number of values")
    if seq_lens is not None and (seq_lens.numel() != B or seq_lens.dtype != torch.int32
                                 or not seq_lens.is_contiguous()):
        raise ValueError("seq_lens must be a contiguous int32 tensor with one length per sequence")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    rc = lib().iq_decode_attention_noalloc(
        q.data_ptr(), _dtype_code(q), k_codes.data_ptr(), k_scales.data_ptr(), v_codes.data_ptr(),
        v_scales.data_ptr(), rot.data_ptr(), 0 if shared_rot else Hkv * ROT_PARAMS,
        seq_lens.data_ptr() if seq_lens is not None else None, B, Hq, Hkv, cap, float(sm_scale), out.data_ptr(),
        HEAD_DIM, BITS, _stream(q))
    _check(rc)
    return out


def decode_attention_multi(q, k_codes, k_scales, v_codes, v_scales, rot, seq_lens=None, sm_scale=0.0,
                           out=None, workspace=None, shared_rot=False):
    """Attention of Q new query tokens per sequence: q [B][Q][Hq][128] (cuda f32/bf16,
    contiguous); the new tokens are the last Q of each sequence's seq_lens cached positions and
    token i attends causally up to its own position.  Other arguments as decode_attention; the
    workspace size is decode_workspace_bytes(B * Q, ...).  Returns out float32 [B][Q][Hq][128]."""
    import torch
    B, Q, Hq, d = q.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    if d != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [B][Q][Hq][128]")
    for t in (k_codes, k_scales, v_codes, v_scales, rot):
        if not t.is_contiguous():
            raise ValueError("cache and rotation tensors must be contiguous")
    for c, sc in ((k_codes, k_scales), (v_codes, v_scales)):
        if tuple(c.shape) != (B, Hkv, cap, RECORD_BYTES) or tuple(sc.shape) != (B, Hkv, cap):
            raise ValueError("caches must be [B][Hkv][cap][48] codes and [B][Hkv][cap] scales")
    if rot.numel() != (Hkv if shared_rot else B * Hkv) * ROT_PARAMS:
        raise ValueError("rot has the wrong number of values")
    if seq_lens is not None and (seq_lens.numel() != B or seq_lens.dtype != torch.int32
                                 or not seq_lens.is_contiguous()):
        raise ValueError("seq_lens must be a contiguous int32 tensor with one length per sequence")
    if out is None:
        out = torch.empty((B, Q, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(B * Q, Hq, Hkv, cap), dtype=torch.uint8, device=q.device)
    rc = lib().iq_decode_attention_multi(
        q.data_ptr(), _dtype_code(q), Q, k_codes.data_ptr(), k_scales.data_ptr(),
        v_codes.data_ptr(), v_scales.data_ptr(), rot.data_ptr(), 0 if shared_rot else Hkv * ROT_PARAMS,
        seq_lens.data_ptr() if seq_lens is not None else None, B, Hq, Hkv, cap, float(sm_scale), out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), HEAD_DIM, BITS, _stream(q))
    _check(rc)
    return out


def decode_attention_append(q, k_new, v_new, positions, k_codes, k_scales, v_codes, v_scales, rot, sm_scale=0.0,
                            out=None, workspace=None, shared_rot=False):
    """One decode step with the new token appended in the same launch: k_new / v_new
    [B][Hkv][128] (cuda f32/bf16, last dim contiguous) are quantised into the cache at
    positions[b] (int32 [B] on the device; outside [0, cap) skips the sequence) and
    attention covers tokens 0..positions[b].  Other arguments as decode_attention.
    Returns out float32 [B][Hq][128]."""
    import torch
    B, Hq, d = q.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    if d != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [B][Hq][128]")
    for t in (k_new, v_new):
        if tuple(t.shape) != (B, Hkv, HEAD_DIM) or t.stride(2) != 1:
            raise ValueError("k_new / v_new must be [B][Hkv][128] with contiguous coordinates")
    if k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must share strides and dtype")
    for t in (k_codes, k_scales, v_codes, v_scales, rot):
        if not t.is_contiguous():
            raise ValueError("cache and rotation tensors must be contiguous")
    for c, sc in ((k_codes, k_scales), (v_codes, v_scales)):
        if tuple(c.shape) != (B, Hkv, cap, RECORD_BYTES) or tuple(sc.shape) != (B, Hkv, cap):
            raise ValueError("caches must be [B][Hkv][cap][48] codes and [B][Hkv][cap] scales")
    if rot.numel() != (Hkv if shared_rot else B * Hkv) * ROT_PARAMS:
        raise ValueError("rot has the wrong number of values")
    if positions.numel() != B or positions.dtype != torch.int32 or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous int32 tensor with one entry per sequence")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, Hq, Hkv, cap)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    rc = lib().iq_decode_attention_append(
        q.data_ptr(), _dtype_code(q), k_new.data_ptr(), v_new.data_ptr(), _dtype_code(k_new),
        k_new.stride(0), k_new.stride(1), positions.data_ptr(),
        k_codes.data_ptr(), k_scales.data_ptr(), v_codes.data_ptr(), v_scales.data_ptr(), rot.data_ptr(),
        0 if shared_rot else Hkv * ROT_PARAMS, B, Hq, Hkv, cap, float(sm_scale), out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), HEAD_DIM, BITS, _stream(q))
    _check(rc)
    return out


def isotropy_workspace_bytes(n_seq, n_heads, n_tokens):
    n = lib().iq_isotropy_workspace_bytes(int(n_seq), int(n_heads), int(n_tokens))
    if n < 0:
        raise IQError(int(n), last_error())
    return int(n)


def isotropy_stats(x, transform, rot=None, dense=None, shared=False, stats=None, workspace=None):
    """Statistics of y = T x over the tokens of every (sequence, head) of x
    [n_seq][n_heads][n_tokens][128] (cuda, f32/bf16, last dim contiguous), for a transform in
    TRANSFORMS.  rot: float32 [n_seq][n_heads][32][8] ("so4", "wht_so4"); dense: float32
    [n_seq][n_heads][128][128] ("dense"); with shared=True both drop the n_seq dimension.
    Returns float64 [n_seq][n_heads][260] on the device (layout in include/iq.h)."""
    import torch
    n_seq, n_heads, n_tokens, d = x.shape
    if d != HEAD_DIM or x.stride(3) != 1:
        raise ValueError("x must be [n_seq][n_heads][n_tokens][128] with contiguous coordinates")
    mode = TRANSFORMS[transform]
    per = n_heads if shared else n_seq * n_heads
    rot_ptr, rot_stride, dense_ptr, dense_stride = None, 0, None, 0
    if transform in ("so4", "wht_so4"):
        if rot is None or rot.numel() != per * ROT_PARAMS or not rot.is_contiguous() or rot.dtype != torch.float32:
            raise ValueError("rot must be a contiguous float32 tensor of %d values" % (per * ROT_PARAMS))
        rot_ptr, rot_stride = rot.data_ptr(), 0 if shared else n_heads * ROT_PARAMS
    if transform == "dense":
        if (dense is None or dense.numel() != per * HEAD_DIM * HEAD_DIM or not dense.is_contiguous()
                or dense.dtype != torch.float32):
            raise ValueError("dense must be a contiguous float32 tensor of %d values" % (per * HEAD_DIM * HEAD_DIM))
        dense_ptr, dense_stride = dense.data_ptr(), 0 if shared else n_heads * HEAD_DIM * HEAD_DIM
    if stats is None:
        stats = torch.empty((n_seq, n_heads, N_STATS), dtype=torch.float64, device=x.device)
    if workspace is None:
        workspace = torch.empty(isotropy_workspace_bytes(n_seq, n_heads, n_tokens), dtype=torch.uint8,
                                device=x.device)
    rc = lib().iq_isotropy_stats(
        x.data_ptr() if n_tokens else None, _dtype_code(x), n_seq, n_heads, n_tokens,
        x.stride(0), x.stride(1), x.stride(2), mode, rot_ptr, rot_stride, dense_ptr, dense_stride,
        stats.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(x))
    _check(rc)
    return stats


# ---------------- measurement: the device's read-only streaming rate ----------------
PROBE_LIB_PATH = os.path.join(_PKG, "libiq_probe.so")
_probe = None


def probe_lib():
    """Load libiq_probe.so (include/iq_probe.h) once: a read-only streaming kernel used to
    measure the HBM read ceiling beside the decode.  Not part of the decode path."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError("libiq_probe.so is not built (%s); run __graft_entry__.build()" % PROBE_LIB_PATH)
        handle = ctypes.CDLL(PROBE_LIB_PATH)
        for name in ("iq_probe_stream_read", "iq_probe_stream_read_nt"):
            getattr(handle, name).restype = ctypes.c_int
            getattr(handle, name).argtypes = [_P, _I64, _I32, _P, _P]
        _probe = handle
    return _probe


def stream_read(buf, sink, n_blocks=2048, nontemporal=False):
    """Read every byte of the cuda tensor buf once (asynchronous, on the current stream); sink
    is a cuda tensor of at least 4 bytes.  nontemporal: loads with the non-temporal hint."""
    name = "iq_probe_stream_read_nt" if nontemporal else "iq_probe_stream_read"
    rc = getattr(probe_lib(), name)(buf.data_ptr(), buf.numel() * buf.element_size(), int(n_blocks),
                                    sink.data_ptr(), _stream(buf))
    if rc != 0:
        raise IQError(rc, name + ": invalid arguments (buf 16-byte aligned, bytes a positive "
                          "multiple of 16, 1 <= n_blocks <= 65535) or launch failure")
