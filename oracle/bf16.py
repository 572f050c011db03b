"""fp32 <-> bfloat16 conversion, round-to-nearest-even (oracle side).

bfloat16 keeps the top 16 bits of an IEEE binary32 value (1 sign, 8 exponent,
7 fraction bits). Rounding a binary32 to it is IEEE round-to-nearest, ties to
even, applied at bit 16; a NaN stays a (quiet) NaN. The pages cast to bf16 in
the Newton-Schulz routine ("Chapter 4: The MuonAdamW Optimizer", section
"bfloat16 and fullgraph Compilation") without naming a rounding mode; this
oracle takes round-to-nearest-even throughout.
"""
import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """binary32 values -> uint16 bfloat16 bit patterns, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    q = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)   # quiet NaN
    return np.where(nan, q, r).astype(np.uint16)


def bf16_bits_to_f32(h) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> binary32 values (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value; the result is returned as float32.

    Input of any float dtype is first rounded to binary32 (as a GPU does when
    it stores an fp32 accumulator), then to bfloat16.
    """
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))
