"""IsoQuant 3-bit KV compression and compressed-space decode attention for
AMD MI355X (gfx950): HIP kernels behind a C ABI (include/iq.h), with a thin
ctypes binding.

Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
Compressed-Space Attention" (arXiv 2608.08081), Abstract.
"""
from .iq import (  # noqa: F401
    IQError, make_rotation, quantize_kv, decode_workspace_bytes, decode_attention, decode_attention_append,
    decode_attention_multi, decode_attention_noalloc, NOALLOC_SCRATCH_BYTES,
    isotropy_workspace_bytes, isotropy_stats, TRANSFORMS, N_STATS, FORMATS, FORMAT_BITS, scale_shape, stream_read,
    lib, LIB_PATH, HEAD_DIM, BITS, RECORD_BYTES, ROT_PARAMS,
)
