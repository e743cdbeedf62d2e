"""fp32 <-> bfloat16 conversion.

bfloat16 is the upper half of an IEEE-754 binary32 word (1 sign bit, 8
exponent bits, 7 fraction bits). The pages use 16-bit parameters and
gradients with fp32 master weights ("第 5 课：ZeRO 与 FSDP", section 2, BF16 +
AdamW; notes on the ZeRO paper, section 2.1, mixed-precision training) but fix
no rounding mode. Reading taken: round to nearest, ties to even; a NaN input
becomes the quiet NaN 0x7FC0 with its sign kept.

Values are carried as uint16 bit patterns.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, as uint16 patterns.

    Adding 0x7FFF plus the lowest kept bit to the 32-bit pattern and dropping
    the low 16 bits rounds the magnitude to nearest with ties to the even
    neighbour; a carry out of the fraction moves into the exponent, which also
    turns values above the largest finite bfloat16 into infinity."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
        rounded = np.where(nan, np.uint16(0x7FC0) | sign, rounded)
    return rounded.astype(np.uint16)
