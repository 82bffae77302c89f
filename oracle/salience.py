"""Element and group salience.  TEST INFRASTRUCTURE (oracle).

Page 1, "核心设计" (core design), component one (SBA): the salience of weight
w_ij is the SparseGPT elimination error, printed as w_ij^2 over the squared
j-th diagonal entry of the inverse Hessian.  Page 2, "Approach": bit-widths
follow the *average* salience of a group.

Readings taken here:

* The inverse is of the damped Hessian H_d = H + damp * mean(diag H) * I with
  damp = 0.01 (the pages are silent on damping; SliM-LLM sits inside GPTQ's
  layer-wise skeleton, which damps the same way).  The undamped H is what the
  Hessian stage returns.
* delta_ij = w_ij^2 / ([H_d^-1]_jj)^2, the squared denominator as printed.
* [H_d^-1]_jj is computed in float64 and stored as float32 (d).  delta is
  then the float32 quantity fl(fl(w*w) / fl(d*d)); the same float32 delta
  weights the SQC error.  Group means are float64 sums of those float32
  values, so the ranking that decides bit-widths is taken from identically
  defined numbers on both sides of a comparison.
* A group is g consecutive input columns across all n rows; S_g is the mean
  of delta over its n*g elements.

Failure convention (LAPACK's): info = j > 0 when the leading minor of order j
of H_d is not positive definite; info = -1 when H or W holds a non-finite
value.  Outputs are unspecified when info != 0.
"""
import numpy as np
from scipy.linalg import lapack

from .decode import as_f32, as_f64


def hinv_diag(H, damp_frac: float = 0.01):
    """(d float64 [m], info): the diagonal of the inverse of the damped Hessian.

    Cholesky (LAPACK potrf) of H_d, then the inverse from that factor (potri);
    both are library primitives used as single steps."""
    h = np.array(H, dtype=np.float64, copy=True)
    m = h.shape[0]
    if not np.all(np.isfinite(h)):
        return np.full(m, np.nan), -1
    h[np.diag_indices(m)] += damp_frac * np.mean(np.diag(h))
    c, info = lapack.dpotrf(h, lower=1, clean=1)
    if info != 0:
        return np.full(m, np.nan), int(info)
    inv, info2 = lapack.dpotri(c, lower=1)
    if info2 != 0:
        return np.full(m, np.nan), int(info2)
    return np.diag(inv).copy(), 0


def element_salience(W, d32) -> np.ndarray:
    """delta [n, m] float32 = fl(fl(w*w) / fl(d*d)), d given as float32."""
    w = as_f32(W)
    d = np.asarray(d32, dtype=np.float32)
    return (w * w) / (d * d)[None, :]


def group_salience(delta32, group: int) -> np.ndarray:
    """S_g [k] float64: mean of delta over the n x g block of column group g."""
    n, m = delta32.shape
    k = m // group
    blocks = delta32.astype(np.float64).reshape(n, k, group)
    return blocks.sum(axis=(0, 2)) / float(n * group)


def salience(H, W, group: int, damp_frac: float = 0.01):
    """(d32 [m] float32, S [k] float64, info) for one linear layer."""
    w = as_f32(W)
    d, info = hinv_diag(H, damp_frac)
    if info == 0 and not np.all(np.isfinite(w)):
        info = -1
    d32 = d.astype(np.float32)
    if info != 0:
        return d32, np.full(w.shape[1] // group, np.nan), info
    S = group_salience(element_salience(w, d32), group)
    return d32, S, 0


__all__ = ["hinv_diag", "element_salience", "group_salience", "salience", "as_f64"]
