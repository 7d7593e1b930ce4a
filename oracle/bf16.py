"""float32 -> bfloat16 rounding (round to nearest, ties to even), test infrastructure.

bfloat16 keeps the top 16 bits of an IEEE binary32 value.  Rounding adds half
an ulp of the kept part (0x7FFF plus the lowest kept bit, so exact ties go to
the even neighbour) to the 32-bit pattern and drops the low 16 bits; a carry
into the exponent gives the next binade or infinity, as it must.  NaN stays NaN.
"""
import numpy as np


def round_f32_to_bf16(x) -> np.ndarray:
    """Return float32 values that are exactly representable in bfloat16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = np.float32("nan")
    return out


def round_to_storage(x, dtype: str) -> np.ndarray:
    """Round float32 results to the cache/storage dtype ('f32' or 'bf16')."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_f32_to_bf16(x)
    if dtype == "f32":
        return x.copy()
    raise ValueError(dtype)
