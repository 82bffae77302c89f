"""Calibration Hessian.  TEST INFRASTRUCTURE (oracle).

Page 1, "核心设计" (core design), component one: the Hessian is approximated
from the calibration activations, with no back-propagation; the FAQ repeats
that calibration needs no gradients.  The pages print the proxy as 2XX^T
(the GPTQ/SparseGPT layer Hessian).

Reading: with activations stored token-major, X[T, m], the proxy is
H = 2 X^T X (the same matrix as 2XX^T for X stored [m, T]), summed over all
calibration tokens, with no 1/T normalisation.  Every use downstream (ranking
of groups, argmin over tau) is invariant to a positive scale of H.
"""
import numpy as np

from .decode import as_f64


def hessian(X) -> np.ndarray:
    """H = 2 X^T X in float64, X token-major [T, m]."""
    x = as_f64(X)
    return 2.0 * (x.T @ x)


def hessian_entries(X, rows, cols) -> np.ndarray:
    """Selected entries H[rows[q], cols[q]] = 2 sum_t X[t, i] X[t, j], one by one."""
    x = as_f64(X)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out = np.empty(len(rows))
    for q, (i, j) in enumerate(zip(rows, cols)):
        out[q] = 2.0 * np.dot(x[:, i], x[:, j])
    return out
