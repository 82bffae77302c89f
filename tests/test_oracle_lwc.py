"""Pins for the oracle's learnable weight clipping (SliM-LLM+; CPU only).

rkmt.cn digest, FAQ on GPTQ / AWQ / OmniQuant (SliM-LLM+ replaces SQC with
OmniQuant's learnable weight clipping); scime.ai summary, opening paragraph
and "Key results" (gradient-based OmniQuant calibration with SBA).

Checks that do not reuse the oracle's own formulas:
* the loss written with H equals the output MSE over the tokens computed
  from X directly (the factor 2T and the orientation of H);
* unit clipping (both sigmoids exactly 1) reproduces the min-max quantizer
  bit for bit;
* the straight-through gradient equals central finite differences of a
  surrogate written independently here (the rounding offsets frozen: a
  weight inside the code range moves as w + delta * s, a clamped one as
  q * s + lo);
* Adam under a constant gradient moves every step by lr * g / (|g| + eps)
  (bias correction exact), and its first two steps worked by hand;
* training lowers the loss from its starting value on an outlier layer.
"""
import numpy as np
import pytest

import oracle
import oracle.lwc as lwc
import synth


def _layer(n=24, m=256, g=64, T=300, seed=3):
    wl = synth.custom(tokens=T, dtype="f32", n=n, m=m, dist="t5", wid=140 + seed, outlier_frac=0.03)
    X, W = synth.make_x(wl, m), synth.make_w(wl, 0)
    H = oracle.hessian(X)
    _, S, info = oracle.salience(H.astype(np.float32), W, g)
    assert info == 0
    bits = oracle.allocation(oracle.rank_groups(S), 1, 2)
    return X, W, H, bits


def test_loss_from_hessian_equals_token_mse():
    X, W, H, bits = _layer()
    rng = np.random.default_rng(0)
    W_hat = (W + 0.01 * rng.standard_normal(W.shape)).astype(np.float32)
    direct = oracle.output_mse(X, W, W_hat)
    via_h = lwc.loss_from_hessian(W, W_hat, H, X.shape[0])
    assert via_h == pytest.approx(direct, rel=1e-10)


def test_unit_clipping_is_minmax():
    _, W, _, bits = _layer()
    n, m = W.shape
    g = 64
    inf = np.full((n, m // g), np.inf)
    s, z, codes, w_hat = lwc.final_quantizer(W, bits, inf, inf, g)
    seg = oracle.as_f32(W).reshape(n, m // g, g)
    s0, z0, maxq = oracle.minmax_params(seg, np.asarray(bits)[None, :])
    q, wh = oracle.fake_quant(seg, s0[..., None], z0[..., None], maxq[..., None])
    np.testing.assert_array_equal(s, s0)
    np.testing.assert_array_equal(z, z0)
    np.testing.assert_array_equal(codes, q.reshape(n, m).astype(np.uint8))
    np.testing.assert_array_equal(w_hat, wh.reshape(n, m))
    # the codes reach both ends of the range in every segment
    c = codes.reshape(n, m // g, g)
    assert np.all(c.min(-1) == 0) and np.all(c.max(-1) == maxq)


def _surrogate_loss(W, H, T, bits, g, gamma, beta, delta, qout, inside):
    """Loss with the rounding frozen at a reference point: inside the code
    range w_hat = w + delta * s, clamped w_hat = q * s + lo."""
    w = oracle.as_f64(W)
    n, m = w.shape
    k = m // g
    seg = w.reshape(n, k, g)
    maxq = 2.0 ** np.asarray(bits, dtype=np.float64) - 1.0
    a = 1.0 / (1.0 + np.exp(-gamma))
    c = 1.0 / (1.0 + np.exp(-beta))
    hi = a * seg.max(-1)
    lo = c * seg.min(-1)
    s = (hi - lo) / maxq[None, :]
    w_hat = np.where(inside, seg + delta * s[..., None], qout * s[..., None] + lo[..., None])
    D = w - w_hat.reshape(n, m)
    return float(np.sum((D @ H) * D) / (2.0 * T))


@pytest.mark.parametrize("init", [4.0, 1.5])
def test_gradient_matches_finite_difference(init):
    X, W, H, bits = _layer()
    T = X.shape[0]
    n, m = W.shape
    g = 64
    k = m // g
    rng = np.random.default_rng(5)
    gamma = init + 0.3 * rng.standard_normal((n, k))
    beta = init + 0.3 * rng.standard_normal((n, k))
    loss, gg, gb = lwc.clip_gradient(W, H, T, bits, gamma, beta, g)
    # the rounding decisions at this point, taken independently
    w = oracle.as_f64(W).reshape(n, k, g)
    maxq = 2.0 ** np.asarray(bits, dtype=np.float64) - 1.0
    a, c = 1 / (1 + np.exp(-gamma)), 1 / (1 + np.exp(-beta))
    hi, lo = a * w.max(-1), c * w.min(-1)
    s = (hi - lo) / maxq[None, :]
    u = w / s[..., None] - lo[..., None] / s[..., None]
    qr = np.rint(u)
    inside = (qr >= 0) & (qr <= maxq[None, :, None])
    delta = qr - u
    qout = np.clip(qr, 0, maxq[None, :, None])
    assert inside.mean() > 0.5
    if init < 3.0:
        assert (~inside).any()        # a clip of ~18%: the clamped branch is exercised too
    assert _surrogate_loss(W, H, T, bits, g, gamma, beta, delta, qout, inside) == pytest.approx(loss, rel=1e-12)
    h = 1e-5
    for (i, j) in [(0, 0), (3, 1), (n - 1, k - 1), (7, 2)]:
        for which, grad in (("gamma", gg), ("beta", gb)):
            e = np.zeros((n, k))
            e[i, j] = h
            gp, bp = (gamma + e, beta) if which == "gamma" else (gamma, beta + e)
            gm, bm = (gamma - e, beta) if which == "gamma" else (gamma, beta - e)
            fd = (_surrogate_loss(W, H, T, bits, g, gp, bp, delta, qout, inside)
                  - _surrogate_loss(W, H, T, bits, g, gm, bm, delta, qout, inside)) / (2 * h)
            assert grad[i, j] == pytest.approx(fd, rel=1e-5, abs=1e-12 * max(1.0, abs(loss))), (which, i, j)


def test_adam_constant_gradient_and_first_steps():
    p = np.zeros(3)
    g = np.array([0.3, -2.0, 1e-3])
    m1, m2 = np.zeros(3), np.zeros(3)
    for t in range(1, 6):
        p_new, m1, m2 = lwc.adam_step(p, g, m1, m2, t, lr=1e-2)
        np.testing.assert_allclose(p_new - p, -1e-2 * g / (np.abs(g) + 1e-8), rtol=1e-12)
        p = p_new
    # first two steps of a changing gradient, worked by hand
    p, m1, m2 = np.zeros(1), np.zeros(1), np.zeros(1)
    p, m1, m2 = lwc.adam_step(p, np.array([0.5]), m1, m2, 1, lr=0.1)
    assert p[0] == pytest.approx(-0.1 * 0.5 / (0.5 + 1e-8), rel=1e-14)
    p, m1, m2 = lwc.adam_step(p, np.array([-0.25]), m1, m2, 2, lr=0.1)
    mh = (0.9 * 0.05 + 0.1 * -0.25) / (1 - 0.81)
    vh = (0.999 * 0.00025 + 0.001 * 0.0625) / (1 - 0.999 ** 2)
    assert p[0] == pytest.approx(-0.1 * 0.5 / (0.5 + 1e-8) - 0.1 * mh / (np.sqrt(vh) + 1e-8), rel=1e-12)


def test_training_lowers_the_loss():
    X, W, H, bits = _layer(n=32, m=256, g=64, T=400, seed=9)
    out = lwc.lwc_calibrate(W, H, X.shape[0], bits, 64, iters=20)
    assert out["loss"].shape == (21,)
    assert out["loss"][-1] < out["loss"][0]
    # the final float32 quantizer's own output error is close to the float64 one
    final = oracle.output_mse(X, W, out["w_hat"])
    assert final == pytest.approx(out["loss"][-1], rel=1e-3)
    assert out["codes"].max() <= 7 and out["scale"].dtype == np.float32
