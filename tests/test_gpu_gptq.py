"""Parity of the GPTQ sweep around the group quantizer (slim_gptq_quantize)
with the oracle, through the C ABI.

Inputs: H, d and the widths are the oracle's (from seeded synthetic X and W),
handed to both sides.  The bar is the integer one: codes, tau indices and
masks bit-equal, scale and zero bit-equal.  Both sides take every decision
in the same arithmetic: the quantizer's float32 sequence on the current
weight rounded to float32, float64 error feedback with the same order inside
a group; only the float64 trailing product after each group sums in another
order (relative differences near 1e-16), so a code could differ only at a
float64 tie.  At full size the oracle runs on sampled rows, which is exact:
given U, each row's sweep depends on that row alone.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TIE, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def slim():
    import post_mixed_precision_amd as s
    s.load_library()
    return s


def _inputs(n, m, g, N, dtype, seed, tokens=512):
    import synth
    wl = synth.custom(tokens=tokens, dtype=dtype, n=n, m=m, dist="t5", wid=80 + seed)
    X, W = synth.make_x(wl, m), synth.make_w(wl, 0)
    H = oracle.hessian(X).astype(np.float32)
    d32, S, info = oracle.salience(H, W, g)
    assert info == 0
    k = m // g
    bits = oracle.allocation(oracle.rank_groups(S), max(1, k // 4), N)
    return H, W, d32, bits


def _run(slim, H, W, bits, d32, g, dtype):
    out = slim.gptq_quantize(torch.from_numpy(H).to("cuda:0"), dev(W, torch, dtype == "bf16"),
                             torch.from_numpy(bits).to("cuda:0"), torch.from_numpy(d32).to("cuda:0"), g)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in out.items()}


def _compare(r, o, g):
    """Exact equality, row by row, up to the first segment where the GPU took
    another calibration decision (tau* or mask) than the oracle.  That segment
    must be a counted near tie (the oracle's best two tau candidates within
    TIE relative, or a weight within TIE sigma of the 3-sigma threshold):
    there the row gets another quantizer, and so other errors for the rest of
    its sweep.  A row whose decisions all agree is compared in full.  Returns
    the number of rows compared in full."""
    n, k = o["scale"].shape
    m = k * g
    tie = (o["gap"] < TIE) | np.any(o["margin"].reshape(n, k, g) < TIE, axis=2)
    words = (o["mask"].reshape(n, m // 32, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(-1)
    words = words.astype(np.uint32)
    rmask = r["mask"].view(np.uint32)
    same = (r["tau_idx"] == o["tau_idx"]) & \
        (rmask.reshape(n, k, g // 32) == words.reshape(n, k, g // 32)).all(axis=2)
    first = np.where((~same).any(axis=1), np.argmax(~same, axis=1), k)
    for i in range(n):
        jq = int(first[i])
        if jq < k:
            assert tie[i, jq], f"row {i}: calibration decision differs at group {jq}, which is not a near tie"
        cq = jq * g
        assert np.array_equal(r["codes"][i, :cq], o["codes"][i, :cq]), f"codes of row {i} before group {jq}"
        assert np.array_equal(r["scale"][i, :jq], o["scale"][i, :jq]), f"scale of row {i}"
        assert np.array_equal(r["zero"][i, :jq], o["zero"][i, :jq]), f"zero of row {i}"
        assert np.array_equal(rmask[i, :cq // 32], words[i, :cq // 32]), f"mask of row {i}"
    full = int(np.sum(first == k))
    print(f"  rows compared in full: {full} of {n} (the rest diverge after a counted near tie)", flush=True)
    return full


@pytest.mark.parametrize("n,m,g,N,dtype", [
    (130, 256, 64, 2, "bf16"),    # ragged row block
    (64, 384, 128, 3, "f32"),
    (200, 96, 32, 2, "f32"),      # m not a multiple of 64: padded factor
    (1, 128, 32, 4, "bf16"),      # one row
    (257, 512, 128, 2, "bf16"),   # several trailing tiles, ragged rows
])
def test_gptq_parity(slim, n, m, g, N, dtype):
    print(f"gptq n={n} m={m} g={g} N={N} {dtype}", flush=True)
    H, W, d32, bits = _inputs(n, m, g, N, dtype, seed=n % 7)
    r = _run(slim, H, W, bits, d32, g, dtype)
    assert int(r["info"][0]) == 0
    o = oracle.gptq_quantize(W, H, bits, d32, g)
    _compare(r, o, g)


def test_gptq_diagonal_hessian_equals_sqc(slim):
    # no column coupling: the sweep must reproduce the plain calibration
    rng = np.random.default_rng(9)
    n, m, g = 96, 256, 64
    H = np.diag(rng.uniform(0.5, 4.0, m)).astype(np.float32)
    W = rng.standard_normal((n, m)).astype(np.float32)
    d32, S, _ = oracle.salience(H, W, g)
    bits = oracle.allocation(oracle.rank_groups(S), 1, 2)
    r = _run(slim, H, W, bits, d32, g, "f32")
    sq = slim.sqc_calibrate(torch.from_numpy(W).to("cuda:0"), torch.from_numpy(bits).to("cuda:0"),
                            torch.from_numpy(d32).to("cuda:0"), g)
    torch.cuda.synchronize()
    assert np.array_equal(r["codes"], host(sq["codes"]))
    assert np.array_equal(r["scale"], host(sq["scale"])) and np.array_equal(r["zero"], host(sq["zero"]))


def test_gptq_failure_codes(slim):
    n, m, g = 8, 64, 32
    W = np.ones((n, m), np.float32)
    bits = np.array([2, 2], np.int8)
    d32 = np.ones(m, np.float32)
    H = -np.eye(m, dtype=np.float32)                 # not positive definite at order 1
    r = _run(slim, H, W, bits, d32, g, "f32")
    assert int(r["info"][0]) == 1
    H = np.eye(m, dtype=np.float32)
    W[3, 5] = np.inf
    r = _run(slim, H, W, bits, d32, g, "f32")
    assert int(r["info"][0]) == -1


def test_gptq_full_size_sampled_rows(slim):
    # the 4096 x 4096 q_proj layer (bf16), H from 8192 of its calibration tokens
    import synth
    wl = synth.WORKLOADS["llama7b-attn-4096"]
    print("gptq 4096 x 4096, H from 8192 tokens", flush=True)
    X = synth.make_x(wl, 4096, 0, 8192)
    W = synth.make_w(wl, 0)
    H = oracle.hessian(X).astype(np.float32)
    d32, S, info = oracle.salience(H, W, 128)
    assert info == 0
    bits = oracle.allocation(oracle.rank_groups(S), 3, 2)
    r = _run(slim, H, W, bits, d32, 128, "bf16")
    assert int(r["info"][0]) == 0
    rows = np.concatenate([np.random.default_rng(11).choice(4096, 30, replace=False), [0, 4095]])
    o = oracle.gptq_quantize(W[rows], H, bits, d32, 128)
    sub = {k: r[k][rows] for k in ("codes", "scale", "zero", "tau_idx", "mask")}
    _compare(sub, o, 128)


def test_salience_u_factor_and_gptq_reuse(slim):
    # slim_salience_u: the salience of slim_salience (float64 rounding in
    # another order) plus U with H_d^-1 = U^T U, checked against LAPACK's
    # factor; slim_gptq_quantize_u on that U must give slim_gptq_quantize's
    # outputs bit for bit (both come from the same reversed sweep of H).
    n, m, g, N = 200, 352, 32, 2          # m not a multiple of 64: padded sweep
    print(f"salience_u / gptq_u n={n} m={m} g={g}", flush=True)
    H, W, d32, bits = _inputs(n, m, g, N, "bf16", seed=5)
    Ht, Wt = torch.from_numpy(H).to("cuda:0"), dev(W, torch, True)
    hinv, gsal, info, _ = slim.salience(Ht, Wt, g)
    hinv_u, gsal_u, info_u, _, U = slim.salience(Ht, Wt, g, want_u=True)
    torch.cuda.synchronize()
    assert int(host(info)[0]) == 0 and int(host(info_u)[0]) == 0
    np.testing.assert_allclose(host(hinv_u), host(hinv), rtol=1e-6)
    np.testing.assert_allclose(host(gsal_u), host(gsal), rtol=1e-9)
    Uh = host(U)
    Uo, inf = oracle.upper_chol_inverse(H)
    assert inf == 0
    assert np.all(np.tril(Uh, -1) == 0.0)
    np.testing.assert_allclose(Uh, Uo, rtol=1e-8, atol=1e-10 * float(np.abs(Uo).max()))
    bt, dt = torch.from_numpy(bits).to("cuda:0"), torch.from_numpy(d32).to("cuda:0")
    r_h = slim.gptq_quantize(Ht, Wt, bt, dt, g)
    r_u = slim.gptq_quantize(None, Wt, bt, dt, g, U=U)
    torch.cuda.synchronize()
    assert int(host(r_u["info"])[0]) == 0
    for key in ("codes", "scale", "zero", "tau_idx", "mask"):
        assert np.array_equal(host(r_u[key]), host(r_h[key])), key
    # a non-finite weight is still reported on this path
    W2 = np.array(W, copy=True)
    W2[7, 11] = 0x7f80                      # bfloat16 +inf
    r2 = slim.gptq_quantize(None, dev(W2, torch, True), bt, dt, g, U=U)
    torch.cuda.synchronize()
    assert int(host(r2["info"])[0]) == -1
