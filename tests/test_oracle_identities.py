"""Pins for the oracle's bfloat16 rounding and for the two identities the SBA
scan kernel is built on (CPU only).

bfloat16 rounding: the trial weights of the SBA search are stored back in the
layer's storage dtype before the trial output is formed (rkmt.cn digest, core
design, component one, read with bfloat16 storage).  ``oracle.bf16_round`` is
checked here against IEEE 754 round-to-nearest-even written out two other
ways: a table of bit patterns worked by hand, and a comparison of the two
neighbouring bfloat16 values in exact arithmetic.

SBA identities (rkmt.cn digest, core design, component one: the balanced
two-pointer scan over [0, k/2] scored by output KL):

* incremental update: step r differs from step r-1 only in the two groups that
  move, so the trial output can be carried from step to step by adding the
  change of those two groups' products;
* chunk-merged KL: the per-token KL of two softmaxes follows from per-chunk
  (max, sum of exponentials) statistics of both outputs and one cross sum,
  merged over chunks by the max-rescale rule.

Each numpy model below is checked against the oracle's direct computation.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


# ---------------------------------------------------------------------------
# bfloat16 rounding
# ---------------------------------------------------------------------------
def _round_bits(u32: int) -> int:
    x = np.array([u32], dtype=np.uint32).view(np.float32)
    return int(oracle.bf16_round(x).view(np.uint32)[0])


# (float32 bits, bfloat16 bits) worked by hand from the definition: keep the
# top 16 bits, and round up (in magnitude) when the dropped 16 bits exceed
# 0x8000, or equal it and the kept last bit is 1.
HAND = [
    (0x3F808000, 0x3F80),   # exact tie, kept last bit even -> stays
    (0x3F818000, 0x3F82),   # exact tie, kept last bit odd -> up to even
    (0x3F808001, 0x3F81),   # just above the tie -> up
    (0x3F807FFF, 0x3F80),   # just below the tie -> down
    (0xBF808000, 0xBF80),   # negative tie, even -> stays (magnitude down)
    (0xBF818000, 0xBF82),   # negative tie, odd -> magnitude up
    (0xBF80C000, 0xBF81),   # negative, above the tie -> magnitude up
    (0x3FFFFFFF, 0x4000),   # rounds up across the binade: just below 2 -> 2
    (0x3FFF8000, 0x4000),   # tie at the top of the binade, odd -> 2
    (0x3F7F8000, 0x3F80),   # tie just below 1, odd -> 1
    (0x00008000, 0x0000),   # subnormal tie, even -> +0
    (0x00018000, 0x0002),   # subnormal tie, odd -> up
    (0x00007FFF, 0x0000),   # smallest subnormals -> +0
    (0x00000001, 0x0000),
    (0x807F8000, 0x8080),   # negative subnormal tie, odd -> smallest normal
    (0x007FFFFF, 0x0080),   # largest subnormal -> smallest normal
    (0x00000000, 0x0000),
    (0x80000000, 0x8000),   # signed zero keeps its sign
    (0x7F7F7FFF, 0x7F7F),   # below the overflow midpoint -> largest finite
    (0x7F7F8000, 0x7F80),   # the overflow midpoint, odd -> infinity
    (0x7F7FFFFF, 0x7F80),   # FLT_MAX -> infinity
    (0xFF7FFFFF, 0xFF80),   # -FLT_MAX -> -infinity
    (0x7F800000, 0x7F80),   # +inf
    (0xFF800000, 0xFF80),   # -inf
]


@pytest.mark.parametrize("src,want", HAND, ids=[f"{s:08x}" for s, _ in HAND])
def test_bf16_round_hand_table(src, want):
    assert _round_bits(src) >> 16 == want
    assert _round_bits(src) & 0xFFFF == 0


@pytest.mark.parametrize("src", [0x7FC00000, 0x7F800001, 0x7FBFFFFF, 0xFFFFFFFF, 0xFF800001, 0x7FFF8000])
def test_bf16_round_nan_stays_nan(src):
    x = np.array([src], dtype=np.uint32).view(np.float32)
    assert np.isnan(oracle.bf16_round(x)[0])


def _bf16_value(b16: int) -> Fraction:
    """Exact value of a finite bfloat16 pattern (or 2^128 for the pattern just
    past the largest finite one, which IEEE rounding treats as the next value)."""
    sign = -1 if b16 & 0x8000 else 1
    e = (b16 >> 7) & 0xFF
    f = b16 & 0x7F
    if e == 0xFF:
        return sign * Fraction(2) ** 128
    if e == 0:
        return sign * Fraction(f, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(f, 128)) * Fraction(2) ** (e - 127)


def _rne_by_comparison(u32: int) -> int:
    """Round-to-nearest-even found by comparing exact distances to the two
    bfloat16 neighbours that bracket the value (truncation and the next one
    away from zero)."""
    x = Fraction(float(np.array([u32], np.uint32).view(np.float32)[0]))
    lo = u32 >> 16                     # truncation toward zero
    hi = lo + 1                        # next pattern away from zero (same sign)
    dl = abs(x - _bf16_value(lo))
    dh = abs(_bf16_value(hi) - x)
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if lo % 2 == 0 else hi   # tie: the even significand


def test_bf16_round_random_against_exact_comparison():
    rng = np.random.default_rng(11)
    # finite patterns of every exponent, both signs; plus low-bit patterns
    # near ties
    u = rng.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]
    near = (rng.integers(0, 2 ** 16, size=500, dtype=np.uint64).astype(np.uint32) << 16) | \
        rng.choice(np.array([0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF], dtype=np.uint32), size=500)
    near = near[((near >> 23) & 0xFF) != 0xFF]
    pats = np.concatenate([u, near])
    got = oracle.bf16_round(pats.view(np.float32)).view(np.uint32)
    assert np.all(got & 0xFFFF == 0)
    want = np.array([_rne_by_comparison(int(p)) for p in pats], dtype=np.uint32)
    np.testing.assert_array_equal(got >> 16, want)


# ---------------------------------------------------------------------------
# SBA: incremental update identity
# ---------------------------------------------------------------------------
def _small_layer(n, m, tokens, wid, dtype="bf16", dist="normal"):
    wl = synth.custom(tokens=tokens, dtype=dtype, n=n, m=m, dist=dist, wid=wid, outlier_frac=0.03)
    return synth.make_x(wl, m), synth.make_w(wl, 0)


def _log_softmax(y):
    mx = y.max(axis=1, keepdims=True)
    return y - (mx + np.log(np.exp(y - mx).sum(axis=1, keepdims=True)))


@pytest.mark.parametrize("n,m,group,N,storage", [
    (48, 512, 64, 2, "bf16"),     # k = 8 (even)
    (40, 448, 64, 3, "bf16"),     # k = 7 (odd: the middle group never moves)
    (32, 384, 128, 2, "f32"),     # k = 3
])
def test_incremental_update_equals_recomputation(n, m, group, N, storage):
    X, W = _small_layer(n, m, 96, wid=300 + m, dtype=storage)
    x = oracle.as_f64(X)
    w = oracle.as_f64(W)
    k = m // group
    _, S, info = oracle.salience(oracle.hessian(X), W, group)
    assert info == 0
    bits_ref, kl_ref, r_ref = oracle.sba_search(X, W, S, N, group, storage)
    order = oracle.rank_groups(S)
    variants = {b: oracle.trial_weights(W, np.full(k, b, np.int8), group, storage).astype(np.float64)
                for b in (N - 1, N, N + 1)}

    lp = _log_softmax(x @ w.T)
    p = np.exp(lp)
    yh = x @ variants[N].T                   # step 0: every group at N bits
    kl = [float((p * (lp - _log_softmax(yh))).sum(1).mean())]
    for r in range(1, k // 2 + 1):
        up, down = int(order[r - 1]), int(order[k - r])
        for gi, b in ((up, N + 1), (down, N - 1)):
            cols = slice(gi * group, (gi + 1) * group)
            yh = yh + x[:, cols] @ (variants[b][:, cols] - variants[N][:, cols]).T
        kl.append(float((p * (lp - _log_softmax(yh))).sum(1).mean()))
    kl = np.array(kl)
    np.testing.assert_allclose(kl, kl_ref, rtol=1e-9, atol=1e-15)
    assert int(np.argmin(kl)) == r_ref
    np.testing.assert_array_equal(oracle.allocation(order, int(np.argmin(kl)), N), bits_ref)


# ---------------------------------------------------------------------------
# SBA: chunk-merged KL identity
# ---------------------------------------------------------------------------
def _chunk_stats(y, yh, chunk):
    """Per output chunk: (M, Z) of y, (Mq, Zq) of yh, S = sum e^{y-M}(y - yh)."""
    out = []
    for c0 in range(0, y.shape[1], chunk):
        a, b = y[:, c0:c0 + chunk], yh[:, c0:c0 + chunk]
        M = a.max(1)
        e = np.exp(a - M[:, None])
        Mq = b.max(1)
        out.append((M, e.sum(1), Mq, np.exp(b - Mq[:, None]).sum(1), (e * (a - b)).sum(1)))
    return out


def _merge_kl(stats):
    """Merge per-chunk statistics by rescaling to the running maximum, then
    KL_t = S/Z - (M + ln Z) + (Mq + ln Zq)."""
    M, Z, Mq, Zq, S = (np.array(v, copy=True) for v in stats[0])
    for Mc, Zc, Mqc, Zqc, Sc in stats[1:]:
        Mn = np.maximum(M, Mc)
        a, b = np.exp(M - Mn), np.exp(Mc - Mn)
        Z, S = Z * a + Zc * b, S * a + Sc * b
        M = Mn
        Mqn = np.maximum(Mq, Mqc)
        Zq = Zq * np.exp(Mq - Mqn) + Zqc * np.exp(Mqc - Mqn)
        Mq = Mqn
    return S / Z - (M + np.log(Z)) + (Mq + np.log(Zq))


@pytest.mark.parametrize("n,chunk", [(512, 128), (300, 128), (96, 32)])
def test_chunk_merged_kl_equals_direct(n, chunk):
    rng = np.random.default_rng(n + chunk)
    m, T = 64, 40
    X = rng.standard_normal((T, m)).astype(np.float32)
    W = (0.3 * rng.standard_normal((n, m))).astype(np.float32)
    # a few outputs far larger than the rest, in one chunk only, so the chunk
    # maxima differ by a wide margin and the rescale matters
    W[chunk // 2: chunk // 2 + 3] *= 12.0
    Wh = (W + 0.05 * rng.standard_normal(W.shape)).astype(np.float32)
    y = X.astype(np.float64) @ W.T.astype(np.float64)
    yh = X.astype(np.float64) @ Wh.T.astype(np.float64)
    kl_direct = oracle.kl_divergence(X, W, Wh, per_token=True)
    kl_merged = _merge_kl(_chunk_stats(y, yh, chunk))
    np.testing.assert_allclose(kl_merged, kl_direct, rtol=1e-9, atol=1e-13)
    # merging in any chunk order gives the same result
    st = _chunk_stats(y, yh, chunk)
    np.testing.assert_allclose(_merge_kl(st[::-1]), kl_direct, rtol=1e-9, atol=1e-13)
