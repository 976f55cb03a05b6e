"""Plain fp64 CPU oracle for IsoQuant compression and compressed-space decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, tables or constants with the HIP path.

Source: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
Compressed-Space Attention" (arXiv 2608.08081), Abstract: IsoQuant applies a
Walsh-Hadamard transform followed by block-diagonal SO(4) rotations before
3-bit scalar quantization (256 stored parameters per head, O(d log d) work),
and attention runs directly on the packed 3-bit tensors without materialising
full-precision KV state.

Every step the pages leave open is a documented reading (see each function's
docstring).  Parity status of each function:
  * hadamard, quat_left, quat_right, block_matrix, rotation_matrix,
    quantize, pack, unpack, decode_attention, multi_token_attention,
    make_rotation: pinned by
    tests/test_oracle_*.py (closed forms, textbook identities, brute force,
    hand-derived golden bytes, published generator test vectors).
  * formats (2- and 4-bit uniform and Lloyd-Max 3-bit quantizers, generic
    packing, attention on them): pinned by tests/test_oracle_formats.py
    (hand-derived records, brute force, Max's published tables).
  * diagnostics.isotropy_stats (the isotropy measures of the rotation and
    its variants): pinned by tests/test_oracle_diagnostics.py (closed-form
    kurtosis values, a hand-worked quantization error, independent
    butterfly / Hamilton-product transforms, a permutation test).
  * The *choice* of reading (Hadamard ordering, quaternion convention,
    quantizer levels, bit layout) cannot be pinned by the pages; parity is
    against these readings.
"""
from .isoquant import (  # noqa: F401
    D, NBLK, LEVELS, RECORD_BYTES,
    bf16_bits_to_f64, hadamard, quat_left, quat_right, quat_conj,
    block_matrix, rotation_matrix, rotate, quantize, dequantize_rotated,
    pack, unpack, decode_attention, multi_token_attention, dense_attention_on_dequantized,
)
from . import diagnostics, formats  # noqa: F401
from .rotation_gen import splitmix64, make_rotation  # noqa: F401
