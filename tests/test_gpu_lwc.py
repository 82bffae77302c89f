"""Parity of SliM-LLM+'s learnable weight clipping (slim_lwc_calibrate) with
the oracle, through the C ABI.

rkmt.cn digest, FAQ on GPTQ / AWQ / OmniQuant (learnable weight clipping in
place of SQC); scime.ai summary, "Key results".

Both sides get the same inputs: the oracle's H rounded to float32, the
widths from the oracle's SBA ranking, the token count.  Both run the same
float64 operations per weight and per segment; only sums (the product D H,
the segment sums, the loss) and the library exp/pow differ in rounding, so
after every Adam step the logits agree to float64 rounding.  The bar:
* loss curve and logits within 1e-9 relative;
* scale and zero bit-equal, except segments whose float64 clipped bound
  lies within 1e-9 relative of the midpoint between two float32 values (there
  the float32 rounding of a bound can go either way: counted as near ties);
* codes equal wherever scale and zero are.
"""
import numpy as np
import pytest

import oracle
import oracle.lwc as lwc
import synth
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def slim():
    import post_mixed_precision_amd as s
    s.load_library()
    return s


def _inputs(n, m, g, N, dtype, T, seed):
    wl = synth.custom(tokens=T, dtype=dtype, n=n, m=m, dist="t5", wid=160 + seed, outlier_frac=0.03, avg_bits=N)
    X, W = synth.make_x(wl, m), synth.make_w(wl, 0)
    H = oracle.hessian(X).astype(np.float32)
    _, S, info = oracle.salience(H, W, g)
    assert info == 0
    k = m // g
    bits = oracle.allocation(oracle.rank_groups(S), max(1, k // 4), N)
    return X, W, H, bits


def _near_f32_midpoint(x64, rel=1e-9):
    """True where a float64 value lies within rel of a float32 rounding midpoint."""
    x = np.asarray(x64, dtype=np.float64)
    f = x.astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    fd = f.astype(np.float64)
    mid = np.where(x >= fd, (fd + up) / 2, (fd + dn) / 2)
    return np.abs(x - mid) <= rel * np.maximum(np.abs(x), 1e-300)


def _compare(r, o, W, bits, g):
    n, m = np.shape(W)
    k = m // g
    lo_err = np.max(np.abs(r["loss"] - o["loss"]) / np.abs(o["loss"]))
    gam, bet = r["logits"][0], r["logits"][1]
    lg_err = max(np.max(np.abs(gam - o["gamma"])), np.max(np.abs(bet - o["beta"])))
    print(f"  loss {o['loss'][0]:.6g} -> {o['loss'][-1]:.6g}; max rel err {lo_err:.2e}; logit err {lg_err:.2e}",
          flush=True)
    assert lo_err <= 1e-9, (r["loss"], o["loss"])
    assert lg_err <= 1e-9 * max(1.0, float(np.max(np.abs(o["gamma"])))), lg_err
    seg = oracle.as_f64(W).reshape(n, k, g)
    hi = lwc.sigmoid(o["gamma"]) * seg.max(-1)
    lo = lwc.sigmoid(o["beta"]) * seg.min(-1)
    tie = _near_f32_midpoint(hi) | _near_f32_midpoint(lo)
    same = (r["scale"] == o["scale"]) & (r["zero"] == o["zero"])
    bad = ~same & ~tie
    assert not bad.any(), f"scale/zero differ at segments {np.argwhere(bad)[:5].tolist()}"
    cg = r["codes"].reshape(n, k, g)
    co = o["codes"].reshape(n, k, g)
    bad_codes = (cg != co).any(-1) & same
    assert not bad_codes.any(), f"codes differ at segments {np.argwhere(bad_codes)[:5].tolist()}"
    print(f"  segments compared exactly: {int(same.sum())} of {n * k} (near ties {int((~same).sum())})", flush=True)


@pytest.mark.parametrize("n,m,g,N,dtype,T,iters", [
    (96, 256, 64, 2, "f32", 300, 20),
    (130, 384, 128, 3, "bf16", 512, 20),   # ragged rows against the 64-row tiles
    (64, 96, 32, 2, "f32", 256, 10),       # m not a multiple of 64: ragged K and columns
    (1, 128, 32, 4, "bf16", 64, 5),        # one row
    (200, 512, 128, 2, "bf16", 1024, 0),   # no step: the starting clipping
])
def test_lwc_parity(slim, n, m, g, N, dtype, T, iters):
    print(f"lwc n={n} m={m} g={g} N={N} {dtype} T={T} iters={iters}", flush=True)
    X, W, H, bits = _inputs(n, m, g, N, dtype, T, seed=n % 11)
    out = slim.lwc_calibrate(dev(W, torch, dtype == "bf16"), torch.from_numpy(bits).to("cuda:0"),
                             torch.from_numpy(H).to("cuda:0"), T, g, iters=iters, want_logits=True)
    torch.cuda.synchronize()
    r = {kk: host(v) for kk, v in out.items()}
    o = lwc.lwc_calibrate(W, H, T, bits, g, iters=iters)
    _compare(r, o, W, bits, g)
    if iters >= 10:
        assert r["loss"][-1] < r["loss"][0]


def test_lwc_packs_and_serves(slim):
    # the learned quantizer's codes pack and serve like SQC's: the packed layer's
    # product equals X W_hat^T of the oracle's dequantized weights
    n, m, g, N, T = 128, 256, 64, 2, 256
    X, W, H, bits = _inputs(n, m, g, N, "f32", T, seed=3)
    out = slim.lwc_calibrate(dev(W, torch, False), torch.from_numpy(bits).to("cuda:0"),
                             torch.from_numpy(H).to("cuda:0"), T, g, iters=10)
    packed, info = slim.pack(out["codes"], torch.from_numpy(bits).to("cuda:0"), g, N)
    xq = torch.from_numpy(X[:4].copy()).to("cuda:0")
    Y = slim.qlinear(xq, packed, torch.from_numpy(bits).to("cuda:0"), out["scale"], out["zero"], g, N)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    from test_gpu_qlinear import _check
    _check(host(Y), X[:4], host(out["codes"]), bits, host(out["scale"]), host(out["zero"]),
           host(packed).view(np.uint32), n, m, g)
