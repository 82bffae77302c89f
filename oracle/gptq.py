"""GPTQ error compensation around the SliM-LLM group quantizer.  TEST INFRASTRUCTURE (oracle).

Page 1 (rkmt.cn digest), "核心设计" (core design) and the FAQ entry on how
SliM-LLM relates to GPTQ / AWQ / OmniQuant: SliM-LLM is a plug-in PTQ
framework built on GPTQ's layer-wise quantization backbone, into which it
inserts its two components (SBA for the group widths, SQC for each group's
quantizer), with groups of 128 columns.  Page 2 (scime.ai), "Builds on":
GPTQ.  The pages do not restate GPTQ itself; its published algorithm
(Frantar et al., "GPTQ: Accurate Post-Training Quantization for Generative
Pre-trained Transformers", ICLR 2023) is:

* quantize the input columns of W one at a time, in order;
* after column c is quantized, move its error onto the columns not yet
  quantized along the optimal-brain-surgeon direction, i.e. with the inverse
  of the Hessian restricted to those columns;
* all those restricted inverses are read off one factor: with H_d^-1 = U^T U
  (U upper triangular, the Cholesky factor of the inverse), the update after
  column c is  e = (w_c - w_hat_c) / U_cc,  W[:, c'] -= e * U[c, c'] for
  c' > c;
* updates of the columns past the current block are batched: the block's
  errors E (n x B) update them at once, W[:, rest] -= E @ U[block, rest].

Readings taken here (the pages only say "GPTQ backbone"):

* H_d = H + damp * mean(diag H) * I with damp = 0.01, the damping the
  salience stage uses, so U and d = diag(H_d^-1) describe one matrix.
* Blocks are the quantization groups.  A group's quantizer is fixed when the
  sweep reaches the group's first column (as GPTQ fixes a group's min-max
  parameters there), and it is SQC's: the 3-sigma mask and tau grid over the
  salience-weighted error, at the group's SBA width, computed on the group's
  current -- already compensated -- weights rounded to float32, with element
  salience from the same float32 d as the rest of the path.
* Each column is then quantized with that quantizer from its current weight
  rounded to float32 (the quantizer's fixed float32 sequence, so the code is
  a float32 decision on both sides of a comparison); the error
  w - w_hat is taken in float64 and all updates are float64.
* Outputs per (row, group): scale, zero, tau index and the 3-sigma mask of
  the calibration; per weight: the code, w_hat = (q - z) s (float32) and the
  propagated error e (float64).
"""
import numpy as np
from scipy.linalg import lapack

from .decode import as_f64
from .quantizer import fake_quant
from .sqc import sqc_calibrate


def upper_chol_inverse(H, damp_frac: float = 0.01):
    """(U float64 [m, m] upper triangular with H_d^-1 = U^T U, info).

    Library primitives as single steps: the Cholesky factor of H_d (potrf),
    the inverse from it (potri, lower triangle, mirrored), then the upper
    Cholesky factor of that inverse (potrf).  info follows LAPACK (j > 0: the
    leading minor of order j is not positive definite; -1: non-finite H)."""
    h = np.array(H, dtype=np.float64, copy=True)
    m = h.shape[0]
    if not np.all(np.isfinite(h)):
        return np.full((m, m), np.nan), -1
    h[np.diag_indices(m)] += damp_frac * np.mean(np.diag(h))
    c, info = lapack.dpotrf(h, lower=1, clean=1)
    if info != 0:
        return np.full((m, m), np.nan), int(info)
    inv, info = lapack.dpotri(c, lower=1)
    if info != 0:
        return np.full((m, m), np.nan), int(info)
    inv = np.tril(inv) + np.tril(inv, -1).T
    u, info = lapack.dpotrf(inv, lower=0, clean=1)
    if info != 0:
        return np.full((m, m), np.nan), int(info)
    return u, 0


def gptq_quantize(W, H, bits, d32, group: int, damp_frac: float = 0.01, lam: float = 0.1, n_tau: int = 50):
    """GPTQ sweep with the SliM-LLM quantizer; see the module docstring.

    W [n, m] (float32, or bfloat16 bit patterns as uint16), H [m, m] the
    undamped Hessian 2 X^T X, bits [k] the group widths, d32 [m] float32
    diag(H_d^-1).  Returns a dict with codes [n, m] uint8, scale / zero
    [n, k] float32, tau_idx [n, k] uint8, mask [n, m] bool, what [n, m]
    float32, err [n, m] float64, gap [n, k] (SQC's relative gap between its
    two best candidates at each calibration), margin [n, m] (each weight's
    distance to the 3-sigma thresholds of its calibration, in sigmas), U and
    info."""
    Wc = as_f64(W).copy()
    n, m = Wc.shape
    k = m // group
    b = np.asarray(bits, dtype=np.int64)
    U, info = upper_chol_inverse(H, damp_frac)
    out = {"U": U, "info": info}
    if info != 0:
        return out
    d32 = np.asarray(d32, dtype=np.float32)
    codes = np.zeros((n, m), dtype=np.uint8)
    what = np.zeros((n, m), dtype=np.float32)
    err = np.zeros((n, m), dtype=np.float64)
    mask = np.zeros((n, m), dtype=bool)
    scale = np.zeros((n, k), dtype=np.float32)
    zero = np.zeros((n, k), dtype=np.float32)
    tau_idx = np.zeros((n, k), dtype=np.uint8)
    gap = np.zeros((n, k))
    margin = np.zeros((n, m))
    for j in range(k):
        c0, c1 = j * group, (j + 1) * group
        # the group's quantizer, on its current weights
        sq = sqc_calibrate(Wc[:, c0:c1].astype(np.float32), b[j:j + 1], d32[c0:c1], group, lam, n_tau)
        s = sq["scale"][:, 0]
        z = sq["zero"][:, 0]
        scale[:, j], zero[:, j], tau_idx[:, j], gap[:, j] = s, z, sq["tau_idx"][:, 0], sq["gap"][:, 0]
        mask[:, c0:c1] = sq["mask_bool"]
        margin[:, c0:c1] = sq["margin"]
        maxq = np.full((n, 1), (1 << int(b[j])) - 1, dtype=np.float32)
        E = np.zeros((n, group))
        for c in range(group):
            col = c0 + c
            q, wh = fake_quant(Wc[:, col].astype(np.float32)[:, None], s[:, None], z[:, None], maxq)
            e = (Wc[:, col] - wh[:, 0].astype(np.float64)) / U[col, col]
            if col + 1 < c1:
                Wc[:, col + 1:c1] -= np.outer(e, U[col, col + 1:c1])
            E[:, c] = e
            codes[:, col] = q[:, 0].astype(np.uint8)
            what[:, col] = wh[:, 0]
        if c1 < m:
            Wc[:, c1:] -= E @ U[c0:c1, c1:]
        err[:, c0:c1] = E
    out.update({"codes": codes, "scale": scale, "zero": zero, "tau_idx": tau_idx, "mask": mask,
                "what": what, "err": err, "gap": gap, "margin": margin})
    return out


__all__ = ["upper_chol_inverse", "gptq_quantize"]
