"""Salience-weighted quantizer calibration (SQC).  TEST INFRASTRUCTURE (oracle).

Page 1, "核心设计" (core design), component two: inside a group, the locally
salient weights are those outside mu +- 3 sigma (about 1% of a group, its
Fig. 4); salient and non-salient weights share one quantizer whose scale and
zero are both scaled by tau, with tau taking linear candidates in
[1 - lambda, 1 + lambda] (lambda = 0.1, n = 50), choosing the candidate with
the smallest l2 reconstruction error and adding no parameters.  Page 2,
"Approach": the calibration is salience-aware.  Page 3 (abstract): it keeps
salient information while minimising error.

Readings taken here:

* Statistics are per segment (one row's g weights in one column group), on
  the weights themselves: mu = mean, sigma = population standard deviation,
  computed in float64; salient set S = {w < mu - 3 sigma} U {w > mu + 3 sigma}
  (strict), U its complement.
* Objective: E(tau) = mean_{i in S}(delta_i e_i^2) + mean_{i in U}(delta_i e_i^2)
  with e_i = w_i - w_hat_i(tau) (float32) and delta_i the float32 element
  salience; products and sums in float64.  The S term is absent when S is
  empty (U is never empty: by Chebyshev |S| <= floor(g/9)).
* tau* is the lowest grid index among the minimisers.  Outputs: scale
  s* = tau* s0, zero z* = tau* z0 (float32), the codes at tau*, the mask
  (bit c of word w of row i = column 32w + c), and the index of tau*.
"""
import numpy as np

from .decode import as_f32
from .quantizer import tau_grid, minmax_params, fake_quant, quant_codes
from .salience import element_salience


def mask_3sigma(seg32):
    """(mask bool, margin float64) over the last axis.

    margin = distance of each weight to the nearer threshold, in units of sigma
    (inf when sigma == 0); used to report near-ties at the threshold."""
    w = np.asarray(seg32, dtype=np.float32).astype(np.float64)
    mu = w.mean(axis=-1, keepdims=True)
    sigma = np.sqrt(((w - mu) ** 2).mean(axis=-1, keepdims=True))
    lo_t = mu - 3.0 * sigma
    hi_t = mu + 3.0 * sigma
    mask = (w < lo_t) | (w > hi_t)
    with np.errstate(divide="ignore", invalid="ignore"):
        margin = np.minimum(np.abs(w - lo_t), np.abs(w - hi_t)) / sigma
    margin = np.where(sigma > 0, margin, np.inf)
    return mask, margin


def _pack_mask(mask_nm: np.ndarray) -> np.ndarray:
    n, m = mask_nm.shape
    b = mask_nm.reshape(n, m // 32, 32).astype(np.uint64)
    sh = np.arange(32, dtype=np.uint64)
    return (b << sh).sum(axis=-1).astype(np.uint32)


def sqc_calibrate(W, bits, d32, group: int, lam: float = 0.1, n_tau: int = 50,
                  rows=None):
    """Calibrate every segment of W (or of the selected ``rows``).

    Returns a dict with scale, zero [n', k] float32; codes [n', m] uint8;
    mask [n', m/32] uint32; tau_idx [n', k] uint8; E [n_tau+1, n', k] float64;
    gap [n', k] (relative gap between the best two E); margin [n', m]."""
    w_all = as_f32(W)
    if rows is not None:
        w_all = w_all[np.asarray(rows)]
    n, m = w_all.shape
    k = m // group
    seg = w_all.reshape(n, k, group)
    b = np.asarray(bits, dtype=np.int64)
    s0, z0, maxq = minmax_params(seg, b[None, :])
    delta = element_salience(w_all, d32).reshape(n, k, group).astype(np.float64)
    mask, margin = mask_3sigma(seg)
    cS = mask.sum(axis=-1)
    cU = group - cS
    taus = tau_grid(lam, n_tau)
    E = np.empty((n_tau + 1, n, k))
    for i, tau in enumerate(taus):
        s = (tau * s0).astype(np.float32)
        z = (tau * z0).astype(np.float32)
        _, wh = fake_quant(seg, s[..., None], z[..., None], maxq[..., None])
        e = (seg - wh).astype(np.float32).astype(np.float64)
        t = delta * (e * e)
        eS = np.where(mask, t, 0.0).sum(axis=-1)
        eU = np.where(mask, 0.0, t).sum(axis=-1)
        E[i] = np.where(cS > 0, eS / np.maximum(cS, 1), 0.0) + eU / cU
    best = np.argmin(E, axis=0)
    tb = taus[best]
    scale = (tb * s0).astype(np.float32)
    zero = (tb * z0).astype(np.float32)
    codes = quant_codes(seg, scale[..., None], zero[..., None], maxq[..., None])
    Es = np.sort(E, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        gap = np.where(Es[0] > 0, (Es[1] - Es[0]) / Es[0], np.where(Es[1] > 0, np.inf, 0.0))
    return {
        "scale": scale, "zero": zero,
        "codes": codes.reshape(n, m).astype(np.uint8),
        "mask": _pack_mask(mask.reshape(n, m)),
        "mask_bool": mask.reshape(n, m),
        "tau_idx": best.astype(np.uint8),
        "E": E, "gap": gap, "margin": margin.reshape(n, m),
    }
