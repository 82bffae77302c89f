"""Pins for the oracle's GPTQ sweep around the SliM-LLM quantizer (CPU only).

rkmt.cn digest, core design and FAQ: SliM-LLM runs inside GPTQ's layer-wise
backbone.  GPTQ (Frantar et al., ICLR 2023) spreads each quantized column's
error over the columns not yet quantized along the inverse of the Hessian
restricted to them, read off the upper Cholesky factor U of H_d^-1.

Checks, each independent of the oracle's own arithmetic:

* U against an explicit inverse, and the GPTQ lemma (row c of U, scaled by
  U_cc, is row 0 of the inverse of the trailing block H_d[c:, c:]);
* a diagonal Hessian couples no columns: the sweep reduces to plain SQC;
* the telescoping identity W - W_hat = E U of the error feedback;
* a brute-force optimal-brain-surgeon sweep that re-inverts the remaining
  Hessian at every column gives the same codes and weights;
* the compensation lowers the layer's output error on a synthetic layer.
"""
import numpy as np
import pytest

import oracle


def _spd(rng, m, t=None):
    t = t or 4 * m
    X = rng.standard_normal((t, m)).astype(np.float32)
    X[:, rng.integers(0, m, 3)] *= 8.0           # a few outlier channels, as in the calibration data
    return oracle.hessian(X), X


def _damped(H, damp=0.01):
    h = np.array(H, dtype=np.float64)
    h[np.diag_indices(h.shape[0])] += damp * np.mean(np.diag(h))
    return h


def test_upper_chol_inverse_against_explicit_inverse_and_lemma():
    rng = np.random.default_rng(1)
    H, _ = _spd(rng, 48)
    U, info = oracle.upper_chol_inverse(H)
    assert info == 0
    assert np.all(np.tril(U, -1) == 0.0) and np.all(np.diag(U) > 0)
    Hi = np.linalg.inv(_damped(H))
    np.testing.assert_allclose(U.T @ U, Hi, rtol=1e-10, atol=1e-12 * np.abs(Hi).max())
    Hd = _damped(H)
    for c in (0, 7, 30, 47):
        Ri = np.linalg.inv(Hd[c:, c:])
        np.testing.assert_allclose(U[c, c:] / U[c, c], Ri[0] / Ri[0, 0], rtol=1e-9, atol=1e-12)
        assert U[c, c] ** 2 == pytest.approx(Ri[0, 0], rel=1e-10)


def test_upper_chol_inverse_failure_codes():
    H = np.eye(8)
    H[3, 3] = np.nan
    assert oracle.upper_chol_inverse(H)[1] == -1
    H = -np.eye(8)
    assert oracle.upper_chol_inverse(H, 0.0)[1] == 1


def test_diagonal_hessian_reduces_to_plain_sqc():
    rng = np.random.default_rng(2)
    n, m, g = 12, 128, 32
    H = np.diag(rng.uniform(0.5, 4.0, m)).astype(np.float32)
    W = rng.standard_normal((n, m)).astype(np.float32)
    d32, S, info = oracle.salience(H, W, g)
    assert info == 0
    bits = oracle.allocation(oracle.rank_groups(S), 1, 2)
    r = oracle.gptq_quantize(W, H, bits, d32, g)
    sq = oracle.sqc_calibrate(W, bits, d32, g)
    assert np.array_equal(r["codes"], sq["codes"])
    assert np.array_equal(r["scale"], sq["scale"]) and np.array_equal(r["zero"], sq["zero"])
    assert np.array_equal(r["tau_idx"], sq["tau_idx"])
    assert np.array_equal(r["mask"], sq["mask_bool"])


def test_error_feedback_identity():
    # w_hat_c = (current w_c) - e_c U_cc and current w_c = w_c - sum_{c'<c} e_c' U[c', c],
    # so W - W_hat = E U exactly (up to float64 rounding), for any H and quantizer.
    rng = np.random.default_rng(3)
    n, m, g = 10, 96, 32
    H, _ = _spd(rng, m)
    W = rng.standard_normal((n, m)).astype(np.float32)
    d32, S, _ = oracle.salience(H, W, g)
    bits = oracle.allocation(oracle.rank_groups(S), 1, 3)
    r = oracle.gptq_quantize(W, H, bits, d32, g)
    lhs = W.astype(np.float64) - r["what"].astype(np.float64)
    rhs = r["err"] @ r["U"]
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(W))


def _obs_brute_force(W, H, bits, d32, g, damp=0.01):
    """GPTQ written as the optimal-brain-surgeon update with the inverse of
    the Hessian of the remaining columns formed explicitly at every column."""
    Wc = W.astype(np.float64).copy()
    n, m = Wc.shape
    Hd = _damped(H, damp)
    codes = np.zeros((n, m), dtype=np.uint8)
    what = np.zeros((n, m), dtype=np.float32)
    for j in range(m // g):
        c0 = j * g
        sq = oracle.sqc_calibrate(Wc[:, c0:c0 + g].astype(np.float32), bits[j:j + 1], d32[c0:c0 + g], g)
        s, z = sq["scale"][:, 0], sq["zero"][:, 0]
        maxq = np.float32((1 << int(bits[j])) - 1)
        for c in range(c0, c0 + g):
            Ri = np.linalg.inv(Hd[c:, c:])
            for i in range(n):
                w32 = np.float32(Wc[i, c])
                q = np.float32(np.rint(np.float32(np.float32(w32 * (np.float32(1) / s[i])) + z[i])))
                q = np.float32(min(max(q, np.float32(0)), maxq))
                wh = np.float32(np.float32(q - z[i]) * s[i])
                codes[i, c], what[i, c] = q, wh
                Wc[i, c + 1:] -= (Wc[i, c] - float(wh)) / Ri[0, 0] * Ri[0, 1:]
    return codes, what


def test_matches_brute_force_obs_sweep():
    rng = np.random.default_rng(4)
    n, m, g = 6, 96, 32
    H, _ = _spd(rng, m)
    W = rng.standard_normal((n, m)).astype(np.float32)
    d32, S, _ = oracle.salience(H, W, g)
    bits = np.array([3, 1, 2], dtype=np.int8)
    r = oracle.gptq_quantize(W, H, bits, d32, g)
    codes, what = _obs_brute_force(W, H, bits, d32, g)
    assert np.array_equal(r["codes"], codes)
    assert np.array_equal(r["what"], what)


def test_compensation_lowers_output_error():
    import synth
    wl = synth.custom(tokens=1024, dtype="f32", n=64, m=256, dist="t5", wid=70)
    X, W = synth.make_x(wl, 256), synth.make_w(wl, 0)
    H = oracle.hessian(X)
    d32, S, info = oracle.salience(H, W, 64)
    assert info == 0
    bits = oracle.allocation(oracle.rank_groups(S), 1, 2)
    r = oracle.gptq_quantize(W, H, bits, d32, 64)
    sq = oracle.sqc_calibrate(W, bits, d32, 64)
    w = oracle.as_f64(W)
    k = 256 // 64
    plain = np.zeros_like(w)
    for j in range(k):
        cols = slice(j * 64, (j + 1) * 64)
        plain[:, cols] = (sq["codes"][:, cols].astype(np.float32) - sq["zero"][:, j:j + 1]) * sq["scale"][:, j:j + 1]
    Hd = np.asarray(H, dtype=np.float64)

    def out_err(Wh):
        D = w - Wh
        return float(np.einsum("ij,jk,ik->", D, Hd, D))

    e_gptq, e_plain = out_err(r["what"].astype(np.float64)), out_err(plain)
    assert e_gptq < 0.95 * e_plain, (e_gptq, e_plain)   # 0.85 on this layer
