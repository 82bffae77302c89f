"""The shared group quantizer and its tau grid.  TEST INFRASTRUCTURE (oracle).

Page 1, "核心设计" (core design), component two (SQC): salient and non-salient
weights of a group share one quantizer whose parameters are scaled by tau
(tau^s for the scale, tau^z for the zero point); tau takes linearly spaced
candidates in [1 - lambda, 1 + lambda] with lambda = 0.1 and n = 50, and the
calibration adds no parameters.  Page 2, "Approach", calls tau a clipping
factor applied to the per-group scale and zero.

Readings taken here (the pages fix neither the quantizer form nor the grid
endpoints' arithmetic):

* Asymmetric uniform quantizer with a float zero point.  For a segment (one
  row's g weights inside one column group) with b bits, maxq = 2^b - 1,
  lo/hi = min/max of the segment:
      s0 = (hi - lo) / maxq,   s0 := 1 if s0 == 0,   z0 = -lo / s0,
      s = tau * s0,  z = tau * z0,  r = 1 / s,
      q = clamp(rint_half_even(w * r + z), 0, maxq),  w_hat = (q - z) * s.
  Every operation is one IEEE float32 operation (no fused multiply-add), in
  exactly this order, so codes are defined to the bit.  At tau = 1 this is
  plain min-max quantization (q(lo) = 0, q(hi) = maxq).
* tau grid: n read as the number of linear steps, giving n + 1 points
  tau_i = 1 + lambda * (2i - n) / n, i = 0..n, evaluated in float64 and
  rounded once to float32; for even n, tau_{n/2} = 1 exactly, so plain
  min-max is always a candidate.
"""
import numpy as np


def tau_grid(lam: float = 0.1, n_tau: int = 50) -> np.ndarray:
    """The n_tau + 1 tau candidates in [1 - lam, 1 + lam], float32."""
    i = np.arange(n_tau + 1, dtype=np.int64)
    t = 1.0 + float(lam) * (2 * i - n_tau).astype(np.float64) / float(n_tau)
    return t.astype(np.float32)


def minmax_params(seg32: np.ndarray, bits):
    """(s0, z0, maxq) float32 over the last axis of ``seg32``; ``bits`` broadcasts
    against the leading axes."""
    seg = np.asarray(seg32, dtype=np.float32)
    lo = seg.min(axis=-1)
    hi = seg.max(axis=-1)
    maxq = (np.left_shift(1, np.asarray(bits, dtype=np.int64)) - 1).astype(np.float32)
    maxq = np.broadcast_to(maxq, lo.shape).astype(np.float32)
    s0 = (hi - lo) / maxq
    s0 = np.where(s0 == np.float32(0), np.float32(1), s0).astype(np.float32)
    z0 = (-lo) / s0
    return s0.astype(np.float32), z0.astype(np.float32), maxq


def quant_codes(seg32, s, z, maxq) -> np.ndarray:
    """Integer codes (float32 holding integers) for the quantizer (s, z, maxq);
    s, z, maxq carry a trailing axis of length 1 against ``seg32``."""
    w = np.asarray(seg32, dtype=np.float32)
    r = np.float32(1) / np.asarray(s, dtype=np.float32)
    t = w * r
    t = t + np.asarray(z, dtype=np.float32)
    q = np.rint(t)
    q = np.minimum(np.maximum(q, np.float32(0)), np.asarray(maxq, dtype=np.float32))
    return q.astype(np.float32)


def fake_quant(seg32, s, z, maxq):
    """(codes, w_hat) float32: quantize then dequantize, w_hat = (q - z) * s."""
    q = quant_codes(seg32, s, z, maxq)
    zz = np.asarray(z, dtype=np.float32)
    wh = (q - zz) * np.asarray(s, dtype=np.float32)
    return q, wh.astype(np.float32)
