"""Pins for the oracle's Hessian and salience stages (CPU only).

Hessian and salience follow page 1 ("SliM-LLM" blog digest), core design,
component one.  The checks below do not re-type the oracle's formulas: they
use brute-force loops, a different LAPACK/numpy routine, closed forms for
diagonal Hessians, and invariances the definitions imply.
"""
import numpy as np
import pytest

import oracle
import synth


def _brute_hessian(x):
    T, m = len(x), len(x[0])
    H = [[0.0] * m for _ in range(m)]
    for i in range(m):
        for j in range(m):
            s = 0.0
            for t in range(T):
                s += x[t][i] * x[t][j]
            H[i][j] = 2.0 * s
    return np.array(H)


def test_hessian_bruteforce_integer_exact():
    rng = np.random.default_rng(1)
    x = rng.integers(-4, 5, size=(23, 7)).astype(np.float32)
    H = oracle.hessian(x)
    assert H.shape == (7, 7)
    np.testing.assert_array_equal(H, _brute_hessian(x.tolist()))


def test_hessian_bf16_storage_and_trace():
    rng = np.random.default_rng(2)
    x = rng.integers(-8, 9, size=(40, 9)).astype(np.float32)
    bits = synth.to_bf16_bits(x)          # small integers are exact in bf16
    H = oracle.hessian(bits)
    np.testing.assert_array_equal(H, _brute_hessian(x.tolist()))
    assert np.allclose(H, H.T)
    assert np.trace(H) == pytest.approx(2.0 * float((x.astype(np.float64) ** 2).sum()))
    assert np.all(np.linalg.eigvalsh(H) > -1e-9 * np.abs(H).max())


def test_hessian_entries_match_bruteforce():
    rng = np.random.default_rng(3)
    x = rng.integers(-3, 4, size=(31, 6)).astype(np.float32)
    Hb = _brute_hessian(x.tolist())
    rows, cols = [0, 5, 2, 3], [0, 1, 2, 5]
    np.testing.assert_array_equal(oracle.hessian_entries(x, rows, cols), Hb[rows, cols])


def test_hinv_diag_vs_numpy_inverse():
    wl = synth.WORKLOADS["tiny-512"]
    X = synth.make_x(wl, 512)
    H = oracle.hessian(X)
    d, info = oracle.hinv_diag(H, 0.01)
    assert info == 0
    Hd = H + 0.01 * np.mean(np.diag(H)) * np.eye(512)
    ref = np.diag(np.linalg.inv(Hd))
    np.testing.assert_allclose(d, ref, rtol=1e-9)


def test_hinv_diag_closed_form_orthogonal_columns():
    # Columns of a scaled Hadamard-like matrix are orthogonal -> H is diagonal,
    # so [H_d^-1]_jj = 1 / (H_jj + damp * mean(diag H)).
    h = np.array([[1.0]])
    for _ in range(4):
        h = np.block([[h, h], [h, -h]])           # 16 x 16 Hadamard
    scales = np.arange(1, 9, dtype=np.float64)
    x = (h[:, :8] * scales[None, :]).astype(np.float32)
    H = oracle.hessian(x)
    diag = 2.0 * 16 * scales ** 2
    np.testing.assert_allclose(H, np.diag(diag), atol=1e-9)
    d, info = oracle.hinv_diag(H, 0.05)
    assert info == 0
    np.testing.assert_allclose(d, 1.0 / (diag + 0.05 * diag.mean()), rtol=1e-12)


def test_hinv_diag_failure_codes():
    H = np.diag([1.0, 1.0, -5.0, 1.0])
    d, info = oracle.hinv_diag(H, 0.01)
    assert info == 3                      # leading minor of order 3 fails
    H2 = np.eye(4)
    H2[1, 2] = np.nan
    _, info2 = oracle.hinv_diag(H2, 0.01)
    assert info2 == -1


def test_element_and_group_salience_closed_form():
    # Diagonal H: d_j = 1/(h_j + a), delta_ij = w_ij^2 (h_j + a)^2.
    h = np.array([2.0, 4.0, 6.0, 8.0])
    a = 0.01 * h.mean()
    W = np.array([[1.0, -2.0, 0.5, 3.0], [0.25, 1.0, -1.0, 2.0]], dtype=np.float32)
    d32, S, info = oracle.salience(np.diag(h), W, group=2, damp_frac=0.01)
    assert info == 0
    np.testing.assert_allclose(d32, 1.0 / (h + a), rtol=1e-7)
    delta = oracle.element_salience(W, d32)
    expect = W.astype(np.float64) ** 2 * (h + a)[None, :] ** 2
    np.testing.assert_allclose(delta, expect, rtol=3e-7)
    # groups {0,1} and {2,3}; mean over the 2 x 2 blocks
    np.testing.assert_allclose(S, [expect[:, :2].mean(), expect[:, 2:].mean()], rtol=3e-7)


def test_salience_invariances():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 64)).astype(np.float32)
    x[:, 40:44] *= 15.0                       # outlier channels in group 2 (g=16)
    W = (rng.standard_normal((24, 64)) * 0.02).astype(np.float32)
    H = oracle.hessian(x)
    _, S, _ = oracle.salience(H, W, 16)
    # permuting rows of W leaves every group mean unchanged
    _, Sp, _ = oracle.salience(H, W[rng.permutation(24)], 16)
    np.testing.assert_allclose(Sp, S, rtol=1e-12)
    # scaling X scales H, hence every delta, by the same factor: same ranking
    _, Sc, _ = oracle.salience(oracle.hessian(x * np.float32(4.0)), W, 16)
    np.testing.assert_array_equal(oracle.rank_groups(Sc), oracle.rank_groups(S))
    # the outlier group is the most salient
    assert oracle.rank_groups(S)[0] == 2


def test_salience_clusters_follow_outlier_channels_tiny():
    wl = synth.WORKLOADS["tiny-512"]
    X, W = synth.make_x(wl, 512), synth.make_w(wl, 0)
    _, S, info = oracle.salience(oracle.hessian(X), W, 128)
    assert info == 0
    ch, _ = synth.outlier_layout(wl, 512)
    hot = sorted(set((ch // 128).tolist()))
    assert sorted(oracle.rank_groups(S)[:len(hot)].tolist()) == hot
