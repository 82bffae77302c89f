"""Storage decoding and bfloat16 rounding for the oracle.  TEST INFRASTRUCTURE.

Layers are stored either as float32 or as bfloat16; this oracle receives
bfloat16 tensors as uint16 bit patterns.  A bfloat16 value is the top 16 bits
of the float32 with the same value, so widening is exact.

``bf16_round`` is used where the method's trial weights are stored back in the
layer's storage dtype before the trial layer output is formed (the reading
that the trial product uses the same operand precision as the layer itself).
It is written from the definition of IEEE round-to-nearest-even onto an 8-bit
significand.
"""
import numpy as np


def _widen_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def as_f32(a) -> np.ndarray:
    """Stored layer tensor -> float32 values."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return _widen_bf16(a)
    return a.astype(np.float32, copy=False)


def as_f64(a) -> np.ndarray:
    """Stored layer tensor -> float64 values (exact)."""
    return as_f32(a).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32.

    Keeps the high 16 bits of the float32 encoding after adding half a unit of
    the kept last place, plus one more if that kept last bit is odd, which is
    round-half-to-even on the dropped 16 bits.  NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32(np.nan)
    return out
