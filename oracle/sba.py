"""Salience-determined bit allocation (SBA).  TEST INFRASTRUCTURE (oracle).

Page 1, "核心设计" (core design), component one:
* bit-widths are allocated so that the KL divergence of the layer output is
  minimal;
* the balance constraint |G_{N-1}| = |G_{N+1}|: when a high-salience group is
  raised to N+1 bits, equally many low-salience groups drop to N-1, so the
  average stays N (2-bit overall becomes a mix of 1, 2 and 3 bits);
* a double-pointer search over the interval [0, k/2] with k = m/128 groups,
  16 iterations for LLaMA-7B.
Page 2, "Approach": groups are ranked by average group salience and the
search is for a KL-optimal ratio with balanced counts.

Readings taken here:

* Ranking: descending S_g, ties broken by the lower group index.
* The two pointers are the two ends of the ranked list.  Step r (0 <= r <=
  floor(k/2)) gives the first r ranked groups N+1 bits, the last r ranked
  groups N-1 bits and the rest N.  Every r is scored (a full scan; for
  m = 4096 and g = 128 that is r = 0 and 16 further steps).  The result is the
  first r with minimal KL.
* A trial allocation is scored with the quantizer at tau = 1 (plain min-max
  per row segment, no mask, no GPTQ error compensation), and the trial weights
  are stored back in the layer's storage dtype (bfloat16 layers round to
  bfloat16) before the output is formed.
* KL objective: for every calibration token t, p_t = softmax over the n
  outputs of x_t W^T and q_t = softmax of x_t W_hat^T; the score is the mean
  over tokens of sum_j p_tj (ln p_tj - ln q_tj), natural log, in float64.

Ablation variants (scime.ai summary, "Measured effects": KL rather than MSE as
the SBA objective, and random or head-tail group allocation instead of SBA;
rkmt.cn digest, Fig. 5 discussion of random and head-tail allocation on OPT):

* MSE objective: the mean over tokens of the squared error of the layer
  output, (1/T) sum_t ||x_t W^T - x_t W_hat^T||^2 (summed over the n outputs),
  in float64.  The pages name the objective only; this is its plainest form.
* Other allocation orders: the salience ranking is replaced by a given order
  of the groups, and the two-pointer scan is otherwise unchanged (step r
  raises the first r groups of the order and lowers the last r).  Head-tail
  is the order of the group index (head groups up, tail groups down); random
  is a seeded permutation.  The scan over r and its objective stay as above,
  so a variant differs from SBA only in which groups move.
"""
import numpy as np

from .decode import as_f32, as_f64, bf16_round
from .quantizer import minmax_params, fake_quant


def rank_groups(S) -> np.ndarray:
    """Group indices by descending salience, ties by ascending index."""
    S = np.asarray(S, dtype=np.float64)
    k = S.shape[0]
    return np.lexsort((np.arange(k), -S))


def allocation(order, r: int, avg_bits: int) -> np.ndarray:
    """Bit-width per group for search step r (int8 [k])."""
    k = len(order)
    assert 0 <= r <= k // 2
    bits = np.full(k, avg_bits, dtype=np.int8)
    if r > 0:
        bits[np.asarray(order[:r])] = avg_bits + 1
        bits[np.asarray(order[k - r:])] = avg_bits - 1
    return bits


def trial_weights(W, bits, group: int, storage: str) -> np.ndarray:
    """Trial-quantized weights (float32 values, [n, m]) at tau = 1 with the
    per-group bit-widths ``bits``, rounded to the storage dtype."""
    w = as_f32(W)
    n, m = w.shape
    k = m // group
    seg = w.reshape(n, k, group)
    s0, z0, maxq = minmax_params(seg, np.asarray(bits)[None, :])
    _, wh = fake_quant(seg, s0[..., None], z0[..., None], maxq[..., None])
    wh = wh.reshape(n, m)
    if storage == "bf16":
        wh = bf16_round(wh)
    return wh


def _log_softmax(y: np.ndarray) -> np.ndarray:
    mx = y.max(axis=1, keepdims=True)
    return y - (mx + np.log(np.exp(y - mx).sum(axis=1, keepdims=True)))


def kl_divergence(X, W, W_hat, per_token: bool = False):
    """Mean over tokens of KL(softmax(x W^T) || softmax(x W_hat^T)), float64."""
    x = as_f64(X)
    lp = _log_softmax(x @ as_f64(W).T)
    lq = _log_softmax(x @ np.asarray(W_hat, dtype=np.float64).T)
    kl_t = (np.exp(lp) * (lp - lq)).sum(axis=1)
    return kl_t if per_token else float(kl_t.mean())


def output_mse(X, W, W_hat, per_token: bool = False):
    """Mean over tokens of ||x W^T - x W_hat^T||^2, float64."""
    x = as_f64(X)
    d = x @ (as_f64(W) - np.asarray(W_hat, dtype=np.float64)).T
    e_t = (d * d).sum(axis=1)
    return e_t if per_token else float(e_t.mean())


def head_tail_order(k: int) -> np.ndarray:
    """Head-tail allocation order: group index order."""
    return np.arange(k, dtype=np.int64)


def random_order(k: int, seed: int) -> np.ndarray:
    """Random allocation order: a permutation from a seeded generator."""
    return np.random.default_rng([seed, 0x5BA]).permutation(k)


def sba_search(X, W, S, avg_bits: int, group: int, storage: str, objective: str = "kl", order=None):
    """(bits int8 [k], score float64 [floor(k/2)+1], r_star) by scoring every step.

    Each step's trial layer output is recomputed from scratch (no reuse of
    earlier steps' products).  ``objective`` is "kl" (the method's) or "mse";
    ``order`` replaces the salience ranking when given (S is then unused)."""
    w = as_f32(W)
    n, m = w.shape
    k = m // group
    order = rank_groups(S) if order is None else np.asarray(order, dtype=np.int64)
    assert sorted(order.tolist()) == list(range(k)), "order must be a permutation of the groups"
    variants = {b: trial_weights(w, np.full(k, b), group, storage)
                for b in (avg_bits - 1, avg_bits, avg_bits + 1)}
    x = as_f64(X)
    y = x @ as_f64(w).T
    if objective == "kl":
        lp = _log_softmax(y)
        p = np.exp(lp)
    elif objective != "mse":
        raise ValueError(objective)
    R = k // 2 + 1
    score = np.empty(R)
    for r in range(R):
        bits = allocation(order, r, avg_bits)
        wh = np.empty((n, m), dtype=np.float32)
        for gi in range(k):
            cols = slice(gi * group, (gi + 1) * group)
            wh[:, cols] = variants[int(bits[gi])][:, cols]
        yh = x @ wh.astype(np.float64).T
        if objective == "kl":
            lq = _log_softmax(yh)
            score[r] = float((p * (lp - lq)).sum(axis=1).mean())
        else:
            d = y - yh
            score[r] = float((d * d).sum(axis=1).mean())
    r_star = int(np.argmin(score))
    return allocation(order, r_star, avg_bits), score, r_star
