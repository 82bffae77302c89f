"""Mixed-precision linear layer from the packed bit-planes.  TEST INFRASTRUCTURE (oracle).

rkmt.cn digest, FAQ on storage and the deployment section: the group-wise
allocation needs no bitmap or codebook, and dequantization keeps the
structure of uniform quantization, so inference reads the packed integer
codes and the per-group scale and zero directly; the digest and the scime.ai
summary ("Limitations"; 61.2 vs 83.9 tokens/s for 2-bit 7B) note the
slowdown of mixed-precision dequantization kernels.

Reading: the layer applied to activations X[t, m] is Y = X W_hat^T with
W_hat[i, c] = (q[i, c] - z[i, c / g]) * s[i, c / g], the dequantization the
calibration defines (one float32 subtraction, then one float32 product), q
decoded from the group-major bit-planes.  The product is taken in float64.
"""
import numpy as np

from .decode import as_f64
from .pack import unpack_bitplanes


def dequant_weights(packed, bits, scale, zero, n: int, m: int, group: int) -> np.ndarray:
    """W_hat float32 [n, m] from the planes and the per-(row, group) scale and zero."""
    q = unpack_bitplanes(packed, bits, n, m, group).astype(np.float32)
    k = m // group
    z = np.repeat(np.asarray(zero, dtype=np.float32).reshape(n, k), group, axis=1)
    s = np.repeat(np.asarray(scale, dtype=np.float32).reshape(n, k), group, axis=1)
    return ((q - z).astype(np.float32) * s).astype(np.float32)


def qlinear(X, packed, bits, scale, zero, n: int, m: int, group: int) -> np.ndarray:
    """Y = X W_hat^T, float64 [t, n]."""
    wh = dequant_weights(packed, bits, scale, zero, n, m, group)
    return as_f64(X) @ wh.astype(np.float64).T
