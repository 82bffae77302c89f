"""Pins for the oracle's mixed-precision linear layer on the packed planes (CPU only).

rkmt.cn digest, FAQ on storage and deployment: no bitmap or codebook, and
dequantization with the structure of uniform quantization.  Checks: a
brute-force loop over unpacked codes, the calibration's own dequantized
weights, and exactness on integer-valued inputs.
"""
import numpy as np
import pytest

import oracle


def _random_layer(rng, n, m, g, N):
    k = m // g
    bits = oracle.allocation(rng.permutation(k), k // 3, N)
    codes = np.zeros((n, m), dtype=np.uint8)
    for j in range(k):
        codes[:, j * g:(j + 1) * g] = rng.integers(0, 2 ** int(bits[j]), size=(n, g))
    scale = (rng.random((n, k)) * 0.01 + 0.001).astype(np.float32)
    zero = (rng.random((n, k)) * 3).astype(np.float32)
    return bits, codes, scale, zero, oracle.pack_bitplanes(codes, bits, g)


def test_qlinear_brute_force():
    rng = np.random.default_rng(21)
    n, m, g, N, t = 5, 96, 32, 2, 3
    bits, codes, scale, zero, packed = _random_layer(rng, n, m, g, N)
    X = rng.standard_normal((t, m)).astype(np.float32)
    Y = oracle.qlinear(X, packed, bits, scale, zero, n, m, g)
    for a in range(t):
        for i in range(n):
            ref = 0.0
            for c in range(m):
                j = c // g
                w = np.float32(np.float32(codes[i, c]) - zero[i, j]) * scale[i, j]
                ref += float(X[a, c]) * float(np.float32(w))
            assert Y[a, i] == pytest.approx(ref, rel=1e-12, abs=1e-12)


def test_qlinear_integer_exact_with_unit_scale():
    rng = np.random.default_rng(22)
    n, m, g, N = 7, 128, 64, 3
    bits, codes, _, _, packed = _random_layer(rng, n, m, g, N)
    k = m // g
    X = rng.integers(-3, 4, size=(2, m)).astype(np.float32)
    Y = oracle.qlinear(X, packed, bits, np.ones((n, k), np.float32), np.zeros((n, k), np.float32), n, m, g)
    np.testing.assert_array_equal(Y, X.astype(np.int64) @ codes.astype(np.int64).T)


def test_qlinear_uses_the_calibrated_weights():
    # The dequantized weights are exactly the SQC calibration's w_hat.
    rng = np.random.default_rng(23)
    n, m, g, N = 16, 256, 128, 2
    W = (rng.standard_normal((n, m)) * 0.02).astype(np.float32)
    d = (rng.random(m) + 0.5).astype(np.float32)
    bits = np.array([3, 1], dtype=np.int8)
    sq = oracle.sqc_calibrate(W, bits, d, g, 0.1, 50)
    packed = oracle.pack_bitplanes(sq["codes"], bits, g)
    wh = oracle.dequant_weights(packed, bits, sq["scale"], sq["zero"], n, m, g)
    seg = W.reshape(n, 2, g)
    maxq = np.array([7, 1], dtype=np.float32)[None, :, None]
    _, wh_ref = oracle.fake_quant(seg, sq["scale"][..., None], sq["zero"][..., None], maxq)
    np.testing.assert_array_equal(wh, wh_ref.reshape(n, m))
