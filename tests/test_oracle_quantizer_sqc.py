"""Pins for the oracle's quantizer, tau grid and SQC stage (CPU only).

SQC follows page 1 ("SliM-LLM" blog digest), core design, component two:
a 3-sigma mask inside each group, and tau in [1 - lambda, 1 + lambda]
(lambda = 0.1, n = 50) scaling scale and zero of one shared quantizer.
Checks use the page constants (tests/golden/pages_constants.json), closed
forms of min-max quantization, Chebyshev's bound, and pure-Python brute force
of the error objective.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))
LAM = GOLD["tau_lambda"]["value"]
NT = GOLD["tau_steps"]["value"]
G = GOLD["group_size"]["value"]


def test_tau_grid_from_pages():
    t = oracle.tau_grid(LAM, NT)
    assert t.dtype == np.float32 and len(t) == NT + 1
    assert t[0] == np.float32(1 - LAM) and t[-1] == np.float32(1 + LAM)
    assert t[NT // 2] == np.float32(1.0)                       # plain min-max is a candidate
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    # each point is rounded once to float32 (half an ulp near 1 is 6e-8)
    np.testing.assert_allclose(np.diff(t.astype(np.float64)), 2 * LAM / NT, rtol=0, atol=1.2e-7)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_minmax_endpoints_and_error_bound(bits):
    rng = np.random.default_rng(bits)
    seg = (rng.standard_normal((200, G)) * 0.02).astype(np.float32)
    s0, z0, maxq = oracle.minmax_params(seg, bits)
    q, wh = oracle.fake_quant(seg, s0[:, None], z0[:, None], maxq[:, None])
    lo_i, hi_i = seg.argmin(1), seg.argmax(1)
    r = np.arange(200)
    assert np.all(q[r, lo_i] == 0) and np.all(q[r, hi_i] == maxq)
    assert np.all(q == np.rint(q)) and q.min() >= 0 and q.max() <= 2 ** bits - 1
    err = np.abs(seg.astype(np.float64) - wh)
    assert np.all(err <= s0[:, None].astype(np.float64) * (0.5 + 1e-5))


def test_one_bit_reconstructs_endpoints():
    rng = np.random.default_rng(7)
    seg = (rng.standard_normal((50, 64))).astype(np.float32)
    s0, z0, maxq = oracle.minmax_params(seg, 1)
    _, wh = oracle.fake_quant(seg, s0[:, None], z0[:, None], maxq[:, None])
    lo, hi = seg.min(1, keepdims=True), seg.max(1, keepdims=True)
    near = np.minimum(np.abs(wh - lo), np.abs(wh - hi))
    assert np.all(near <= 4 * np.spacing(np.maximum(np.abs(lo), np.abs(hi))))


def test_constant_segment_is_finite_and_exact():
    seg = np.full((3, 32), -0.75, dtype=np.float32)
    s0, z0, maxq = oracle.minmax_params(seg, 2)
    assert np.all(s0 == 1)
    q, wh = oracle.fake_quant(seg, s0[:, None], z0[:, None], maxq[:, None])
    assert np.all(q == 0) and np.all(wh == np.float32(-0.75))


def test_round_half_even():
    seg = np.array([[0.0, 0.5, 1.5, 2.5, 3.0]], dtype=np.float32)
    q = oracle.quant_codes(seg, np.float32([[1.0]]), np.float32([[0.0]]), np.float32([[3.0]]))
    np.testing.assert_array_equal(q[0], [0, 0, 2, 2, 3])


def test_quantizer_matches_scalar_float32_loop():
    rng = np.random.default_rng(11)
    seg = (rng.standard_t(5, size=(6, 32)) * 0.02).astype(np.float32)
    for bits in (1, 2, 3):
        s0, z0, maxq = oracle.minmax_params(seg, bits)
        for tau in oracle.tau_grid(LAM, NT)[::7]:
            s = (tau * s0).astype(np.float32)
            z = (tau * z0).astype(np.float32)
            q, wh = oracle.fake_quant(seg, s[:, None], z[:, None], maxq[:, None])
            for i in range(6):
                one = np.float32(1)
                r = one / s[i]
                for c in range(32):
                    t = np.float32(seg[i, c] * r)
                    t = np.float32(t + z[i])
                    qq = min(max(float(np.rint(t)), 0.0), float(maxq[i]))
                    w_h = np.float32(np.float32(np.float32(qq) - z[i]) * s[i])
                    assert q[i, c] == qq and wh[i, c] == w_h


def test_mask_planted_outlier():
    a = 0.01
    seg = np.array([a if i % 2 else -a for i in range(127)] + [20 * a], dtype=np.float32)
    mask, _ = oracle.mask_3sigma(seg[None, :])
    assert mask[0].tolist() == [False] * 127 + [True]


def test_mask_equally_spaced_is_empty():
    seg = np.linspace(-1, 1, G).astype(np.float32)
    mask, margin = oracle.mask_3sigma(seg[None, :])
    assert not mask.any()
    z = (seg - seg.mean()) / seg.std()
    assert abs(z).max() == pytest.approx(math.sqrt(3) * 127 / math.sqrt(128 * 128 - 1) * math.sqrt(128 / 128), rel=1e-2)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_mask_chebyshev_bound(g):
    rng = np.random.default_rng(g)
    seg = (rng.standard_t(2, size=(4000, g))).astype(np.float32)
    seg[::7, 0] = 1e3                                    # extreme single outliers
    mask, _ = oracle.mask_3sigma(seg)
    assert mask.sum(1).max() <= g // 9


def test_mask_fraction_student_t_near_one_percent():
    rng = np.random.default_rng(0)
    seg = (rng.standard_t(5, size=(20000, G)) * 0.02).astype(np.float32)
    mask, _ = oracle.mask_3sigma(seg)
    frac = mask.mean()
    assert 0.003 < frac < 0.03        # pages: about 1% of a group


def _brute_E(w, delta, bits, taus):
    """Pure-Python E(tau) for one segment: mean over S plus mean over U."""
    g = len(w)
    mu = sum(float(v) for v in w) / g
    sd = math.sqrt(sum((float(v) - mu) ** 2 for v in w) / g)
    S = [i for i in range(g) if float(w[i]) < mu - 3 * sd or float(w[i]) > mu + 3 * sd]
    U = [i for i in range(g) if i not in S]
    s0, z0, maxq = oracle.minmax_params(np.asarray(w)[None, :], bits)
    out = []
    for tau in taus:
        s = np.float32(tau * s0[0])
        z = np.float32(tau * z0[0])
        r = np.float32(1) / s
        e2 = []
        for v in w:
            t = np.float32(np.float32(v * r) + z)
            q = np.float32(min(max(float(np.rint(t)), 0.0), float(maxq[0])))
            e = np.float32(v - np.float32(np.float32(q - z) * s))
            e2.append(float(e) * float(e))
        eS = sum(float(delta[i]) * e2[i] for i in S) / len(S) if S else 0.0
        eU = sum(float(delta[i]) * e2[i] for i in U) / len(U)
        out.append(eS + eU)
    return np.array(out), S


def test_sqc_bruteforce_and_never_worse_than_minmax():
    rng = np.random.default_rng(21)
    n, m, g = 3, 64, 32
    W = (rng.standard_t(4, size=(n, m)) * 0.02).astype(np.float32)
    W[1, 5] = 0.3                                            # a local outlier
    d32 = (1.0 / (1.0 + rng.random(m))).astype(np.float32)
    bits = np.array([1, 3], dtype=np.int8)
    res = oracle.sqc_calibrate(W, bits, d32, g, LAM, NT)
    taus = oracle.tau_grid(LAM, NT)
    delta = oracle.element_salience(W, d32)
    one = int(np.argmin(np.abs(taus - 1)))
    for i in range(n):
        for j in range(m // g):
            cols = slice(j * g, (j + 1) * g)
            E, S = _brute_E(W[i, cols], delta[i, cols], int(bits[j]), taus)
            np.testing.assert_allclose(res["E"][:, i, j], E, rtol=1e-12, atol=0)
            assert res["tau_idx"][i, j] == int(np.argmin(E))
            assert E[res["tau_idx"][i, j]] <= E[one]
            mrow = res["mask_bool"][i, cols]
            assert sorted(np.nonzero(mrow)[0].tolist()) == S
    assert res["mask_bool"][1, 5]
    # outputs are consistent with the chosen tau
    s0, z0, _ = oracle.minmax_params(W.reshape(n, 2, g), bits[None, :])
    np.testing.assert_array_equal(res["scale"], (taus[res["tau_idx"]] * s0).astype(np.float32))
    np.testing.assert_array_equal(res["zero"], (taus[res["tau_idx"]] * z0).astype(np.float32))


def test_sqc_mask_words_layout():
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((2, 64)) * 0.02).astype(np.float32)
    W[0, 33] = 1.0
    W[1, 2] = -1.0
    res = oracle.sqc_calibrate(W, np.array([2, 2]), np.ones(64, np.float32), 32, LAM, NT)
    assert res["mask"].shape == (2, 2)
    assert res["mask"][0, 1] & (1 << 1)
    assert res["mask"][1, 0] & (1 << 2)
