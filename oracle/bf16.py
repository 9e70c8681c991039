"""float32 -> bfloat16 rounding for the oracle (test infrastructure only).

The pages keep weights and gradients in BF16 and the Adam state (master
copy, m, v) in FP32, at 16 bytes per parameter (lilting.ch article, section
"LLM訓練のメモリを分解する", the per-parameter byte table).  After the FP32
update the BF16 weight is refreshed from the master; the rounding used here is
IEEE round-to-nearest, ties-to-even, on the 16 dropped mantissa bits.  NaN
inputs map to a quiet NaN with the sign kept.

Pinned by tests/test_oracle_bf16.py against a definition that never touches
the bit trick: pick the nearer of the two neighbouring bf16 values computed in
float64, ties to the even one.
"""
import numpy as np


def bf16_bits(x):
    """Return the bf16 bit patterns (uint16) of float32 ``x``, rounded RNE."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    quiet_nan = ((u >> 16) | 0x0040) & 0xFFFF
    return np.where(is_nan, quiet_nan, rounded).astype(np.uint16)


def bf16_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_bf16(x):
    """Round float32 ``x`` to the nearest bf16 value (RNE); returns float32."""
    return bf16_to_f32(bf16_bits(x))
