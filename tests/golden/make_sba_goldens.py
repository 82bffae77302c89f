"""Write the oracle's SBA scan results for the full-size layers to JSON.

    python tests/golden/make_sba_goldens.py [attn-full] [mlp70b-slice] [mlp70b-batches] [mlp13b-full-width]

Every stored value comes from the CPU oracle (``oracle/``) on the seeded
synthetic inputs (``synth/``); nothing here touches the GPU path.  The scan
objective is a mean over tokens of a per-token quantity, so a long token range
is scored chunk by chunk with ``oracle.sba_search`` and the chunk curves are
combined with token-count weights; that is the same mean, summed in another
order.  The group salience S handed to the scan is the oracle's, from a
Hessian over the first tokens of the layer's calibration set (rounded to
float32, the dtype the GPU's Hessian is stored in); it is stored with the
result so the GPU test can hand the very same S to its scan.

Sources: rkmt.cn digest, core design, component one (balanced two-pointer
scan over [0, k/2] scored by output KL; 16 steps for LLaMA-7B); evaluation
protocol (128 x 2048 calibration tokens).
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402


def _scan_over(wl, W, S, N, g, t0, t1, chunk):
    """Token-weighted mean of the oracle's per-chunk scan curves over [t0, t1)."""
    m = W.shape[1]
    acc = None
    for a in range(t0, t1, chunk):
        b = min(t1, a + chunk)
        X = synth.make_x(wl, m, a, b)
        _, kl, _ = oracle.sba_search(X, W, S, N, g, wl.dtype)
        acc = kl * (b - a) if acc is None else acc + kl * (b - a)
        print(f"  tokens [{a}, {b}) done", flush=True)
    return acc / (t1 - t0)


def _salience(wl, W, g, h_tokens):
    X = synth.make_x(wl, W.shape[1], 0, h_tokens)
    H = oracle.hessian(X).astype(np.float32)
    d, S, info = oracle.salience(H, W, g, 0.01)
    assert info == 0
    return S


def _write(name, rec):
    rec["command"] = f"python tests/golden/make_sba_goldens.py {name}"
    path = os.path.join(HERE, f"sba_{name}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"wrote {path}", flush=True)


def make(name, wname, idx, g, h_tokens, t0, t1, chunk):
    wl = synth.WORKLOADS[wname]
    lin = wl.linears[idx]
    N = wl.avg_bits
    T = wl.tokens
    t0 = t0 if t0 >= 0 else T + t0
    t1 = t1 if t1 > 0 else T + t1
    print(f"{name}: {wname}/{lin.name} {lin.n}x{lin.m} g={g} N={N} tokens [{t0}, {t1})", flush=True)
    start = time.time()
    W = synth.make_w(wl, idx)
    S = _salience(wl, W, g, h_tokens)
    kl = _scan_over(wl, W, S, N, g, t0, t1, chunk)
    order = oracle.rank_groups(S)
    r_star = int(np.argmin(kl))
    bits = oracle.allocation(order, r_star, N)
    s_sorted = np.sort(kl)
    rec = {
        "workload": wname, "linear": lin.name, "n": lin.n, "m": lin.m, "group": g, "avg_bits": N,
        "storage": wl.dtype, "seed": 0, "hessian_tokens": [0, h_tokens], "tokens": [t0, t1],
        "group_sal": [float(v) for v in S],
        "kl": [float(v) for v in kl], "r_star": r_star, "bits": [int(b) for b in bits],
        "best_two_rel_gap": float((s_sorted[1] - s_sorted[0]) / s_sorted[0]),
        "oracle_seconds": round(time.time() - start, 1),
    }
    _write(name, rec)


JOBS = {
    # the 4096 x 4096 attention projection over all 262144 calibration tokens
    "attn-full": ("llama7b-attn-4096", 0, 128, 8192, 0, 0, 4096),
    # the 28672 x 8192 MLP on its last 256 calibration tokens
    "mlp70b-slice": ("large-13b-70b", 1, 128, 2048, -256, 0, 256),
    # the 28672 x 8192 MLP on 2048 tokens that straddle the boundary between
    # the first two 32768-token statistics batches of the full-token scan
    "mlp70b-batches": ("large-13b-70b", 1, 128, 2048, 32768 - 1024, 32768 + 1024, 512),
    # the 13824 x 5120 MLP over 8192 tokens
    "mlp13b-full-width": ("large-13b-70b", 0, 128, 2048, 0, 8192, 2048),
}


if __name__ == "__main__":
    names = sys.argv[1:] or list(JOBS)
    for nm in names:
        make(nm, *JOBS[nm])
