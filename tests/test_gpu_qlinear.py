"""Parity of the mixed-precision linear layer on the packed planes (slim_qlinear)
with the oracle, through the C ABI: decode batches (t <= 8: nibble tables and
the small matrix-core kernel) and prefill batches (t > 8: the GEMM over the
planes).

Inputs are drawn by the test (codes per group width, scale, zero, X) or come
from the oracle's calibration and packing; the oracle dequantizes and forms
the product in float64.  Tolerance, from the arithmetic: the kernel sums in
float32 the masked X values, the planes and the groups, and subtracts the
zero term per group, so each output is compared within 3e-5 of
sum_c |x_c| (q_ic + |z|) s (the magnitudes it adds).
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def slim():
    import post_mixed_precision_amd as s
    s.load_library()
    return s


def _layer(seed, n, m, g, N):
    rng = np.random.default_rng(seed)
    k = m // g
    bits = oracle.allocation(rng.permutation(k), k // 3, N)
    codes = np.zeros((n, m), dtype=np.uint8)
    for j in range(k):
        codes[:, j * g:(j + 1) * g] = rng.integers(0, 2 ** int(bits[j]), size=(n, g), dtype=np.uint8)
    scale = (rng.random((n, k)) * 0.01 + 1e-3).astype(np.float32)
    zero = (rng.random((n, k)) * (2.0 ** bits[None, :].astype(np.float32))).astype(np.float32)
    return bits, codes, scale, zero, oracle.pack_bitplanes(codes, bits, g)


def _x(seed, t, m, dtype):
    X = np.random.default_rng(seed).standard_normal((t, m)).astype(np.float32)
    import synth
    return synth.to_bf16_bits(X) if dtype == "bf16" else X


def _run(slim, X, packed, bits, scale, zero, g, N, dtype):
    Y = slim.qlinear(dev(X, torch, dtype == "bf16"), torch.from_numpy(packed.view(np.int32)).to("cuda:0"),
                     torch.from_numpy(bits).to("cuda:0"), torch.from_numpy(scale).to("cuda:0"),
                     torch.from_numpy(zero).to("cuda:0"), g, N)
    torch.cuda.synchronize()
    return host(Y)


def _check(Yg, X, codes, bits, scale, zero, packed, n, m, g):
    import synth
    Yo = oracle.qlinear(X, packed, bits, scale, zero, n, m, g)
    k = m // g
    xa = np.abs(synth.as_float(X).astype(np.float64))
    mag = np.zeros((n, m))
    for j in range(k):
        cols = slice(j * g, (j + 1) * g)
        mag[:, cols] = (codes[:, cols] + np.abs(zero[:, j:j + 1])) * scale[:, j:j + 1]
    bound = 3e-5 * (xa @ mag.T) + 1e-30
    err = np.abs(Yg.astype(np.float64) - Yo)
    assert np.all(err <= bound), float(np.max(err / bound))


@pytest.mark.parametrize("t,n,m,g,N,dtype", [
    (1, 300, 512, 128, 2, "bf16"),     # ragged row block
    (3, 130, 256, 64, 3, "f32"),
    (8, 64, 96, 32, 2, "bf16"),        # one plane word per row segment, odd k
    (5, 257, 384, 128, 2, "f32"),
    (2, 1000, 2048, 128, 4, "bf16"),   # several runs of groups
])
def test_qlinear_parity(slim, t, n, m, g, N, dtype):
    print(f"qlinear t={t} n={n} m={m} g={g} N={N} {dtype}", flush=True)
    bits, codes, scale, zero, packed = _layer(n + m, n, m, g, N)
    X = _x(t + m, t, m, dtype)
    _check(_run(slim, X, packed, bits, scale, zero, g, N, dtype), X, codes, bits, scale, zero, packed, n, m, g)


@pytest.mark.parametrize("t,n,m,g,N,dtype", [
    (9, 64, 256, 128, 4, "bf16"),      # the smallest prefill batch; widths 3..5
    (16, 300, 512, 128, 2, "bf16"),    # ragged row tile
    (129, 200, 256, 64, 3, "f32"),     # ragged token tile; float32 X as three bfloat16 terms
    (300, 130, 384, 32, 2, "bf16"),    # one plane word per row segment
    (40, 96, 256, 64, 7, "f32"),       # widths 6..8: the byte conversion of the codes
    (512, 1024, 1024, 128, 2, "bf16"), # several tiles both ways
])
def test_qlinear_prefill_parity(slim, t, n, m, g, N, dtype):
    # t > 8: the GEMM over the planes
    print(f"qlinear prefill t={t} n={n} m={m} g={g} N={N} {dtype}", flush=True)
    bits, codes, scale, zero, packed = _layer(n + m + t, n, m, g, N)
    X = _x(t + 2 * m, t, m, dtype)
    _check(_run(slim, X, packed, bits, scale, zero, g, N, dtype), X, codes, bits, scale, zero, packed, n, m, g)


def test_qlinear_prefill_70b_sampled_rows(slim):
    # the 70B-shaped MLP (28672 x 8192) at 256 tokens, sampled rows against the
    # float64 product of the dequantized weights; and every row of the batch
    # against the decode kernel's one-token result for that row
    print("qlinear prefill 28672 x 8192, t = 256", flush=True)
    bits, codes, scale, zero, packed = _layer(13, 28672, 8192, 128, 2)
    X = _x(14, 256, 8192, "bf16")
    Y = _run(slim, X, packed, bits, scale, zero, 128, 2, "bf16")
    rows = np.concatenate([np.random.default_rng(6).choice(28672, 29, replace=False), [0, 28671]])
    import synth
    xf = synth.as_float(X).astype(np.float64)
    q = codes[rows].astype(np.float32)
    z = np.repeat(zero[rows], 128, axis=1)
    sc = np.repeat(scale[rows], 128, axis=1)
    Wh = ((q - z).astype(np.float32) * sc).astype(np.float32).astype(np.float64)
    mag = np.abs(xf) @ ((q + np.abs(z)) * sc).astype(np.float64).T
    err = np.abs(Y[:, rows].astype(np.float64) - xf @ Wh.T)
    assert np.all(err <= 3e-5 * mag + 1e-30), float(np.max(err / (3e-5 * mag + 1e-30)))
    for a in (0, 100, 255):
        Y1 = _run(slim, X[a:a + 1], packed, bits, scale, zero, 128, 2, "bf16")
        np.testing.assert_allclose(Y[a], Y1[0], rtol=1e-5, atol=1e-5 * float(np.abs(Y1).max()))


def test_qlinear_on_calibrated_layer(slim):
    # codes, scale and zero from the oracle's calibration of a synthetic layer
    import synth
    wl = synth.custom(tokens=256, dtype="bf16", n=192, m=512, dist="t5", wid=60)
    X, W = synth.make_x(wl, 512), synth.make_w(wl, 0)
    d, S, _ = oracle.salience(oracle.hessian(X), W, 128)
    bits = oracle.allocation(oracle.rank_groups(S), 1, 2)
    sq = oracle.sqc_calibrate(W, bits, d, 128, 0.1, 50)
    packed = oracle.pack_bitplanes(sq["codes"], bits, 128)
    Xt = X[:4]
    Yg = _run(slim, Xt, packed, bits, sq["scale"], sq["zero"], 128, 2, "bf16")
    _check(Yg, Xt, sq["codes"], bits, sq["scale"], sq["zero"], packed, 192, 512, 128)


def test_qlinear_full_size_and_batch_consistency(slim):
    # 4096 x 4096 at 2 bits against the oracle; the 70B-shaped MLP on sampled
    # rows and on properties: every row of an 8-token batch agrees with the single-token
    # result (the batch size sets how many groups one workgroup sums, so only
    # the float32 order of the group sums differs), and the product is
    # linear in X.
    print("qlinear 4096 x 4096, t = 1 and 8", flush=True)
    bits, codes, scale, zero, packed = _layer(1, 4096, 4096, 128, 2)
    X = _x(2, 8, 4096, "bf16")
    Yg = _run(slim, X, packed, bits, scale, zero, 128, 2, "bf16")
    _check(Yg, X, codes, bits, scale, zero, packed, 4096, 4096, 128)
    print("qlinear 28672 x 8192 (70B MLP shape), t = 1 and 8", flush=True)
    bits, codes, scale, zero, packed = _layer(3, 28672, 8192, 128, 2)
    X = np.random.default_rng(4).standard_normal((8, 8192)).astype(np.float32)
    Y8 = _run(slim, X, packed, bits, scale, zero, 128, 2, "f32")
    # sampled rows (the last row block's tail included) against the float64
    # product of the dequantized weights, as the oracle forms it
    rows = np.concatenate([np.random.default_rng(5).choice(28672, 61, replace=False), [0, 28670, 28671]])
    q = codes[rows].astype(np.float32)
    z = np.repeat(zero[rows], 128, axis=1)
    sc = np.repeat(scale[rows], 128, axis=1)
    Wh = ((q - z).astype(np.float32) * sc).astype(np.float32).astype(np.float64)
    Yo = X.astype(np.float64) @ Wh.T
    mag = np.abs(X.astype(np.float64)) @ ((q + np.abs(z)) * sc).astype(np.float64).T
    err = np.abs(Y8[:, rows].astype(np.float64) - Yo)
    assert np.all(err <= 3e-5 * mag + 1e-30), float(np.max(err / (3e-5 * mag + 1e-30)))
    del codes
    for a in (0, 5, 7):
        Y1 = _run(slim, X[a:a + 1], packed, bits, scale, zero, 128, 2, "f32")
        np.testing.assert_allclose(Y1[0], Y8[a], rtol=1e-5, atol=1e-5 * float(np.abs(Y8[a]).max()))
    Ys = _run(slim, X[:1] + X[1:2], packed, bits, scale, zero, 128, 2, "f32")
    np.testing.assert_allclose(Ys[0], Y8[0] + Y8[1], rtol=1e-4, atol=1e-4 * float(np.abs(Y8[:2]).max()))


def test_qlinear_bad_widths_give_nan(slim):
    n, m, g = 64, 256, 128
    bits = np.array([3, 3], dtype=np.int8)           # sums to 6, not 2 * 2
    packed = np.zeros(n * m * 2 // 32, dtype=np.uint32)
    scale = np.ones((n, 2), np.float32)
    zero = np.zeros((n, 2), np.float32)
    Y = _run(slim, np.ones((1, m), np.float32), packed, bits, scale, zero, g, 2, "f32")
    assert np.all(np.isnan(Y))
