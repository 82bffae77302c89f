"""Throughput of the SliM-LLM per-layer quantizer path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--linear I]

A step is one pass of the whole path over one linear layer whose inputs are
already resident in HBM: Hessian 2X^TX, damped inverse-diagonal salience and
group means, the SBA scan scored by output KL, SQC calibration and bit-plane
packing.  The default workload is the largest single layer, the
Llama-70B-shaped MLP projection: W 28672 x 8192 bf16 ~ N(0, 0.015^2), X 262144
calibration tokens (128 sequences of 2048) x 8192 bf16 with 1% clustered
outlier channels, group 128, 2-bit average over {1, 2, 3}; synthetic, seeded
(synth/).  value = n*m / 1e6 / seconds per step (Mparams quantized per
second).  --workload llama7b-attn-4096 --linear 0 gives the 4096 x 4096
attention projection; --decoder-layer times a whole 7B-shaped decoder layer
(seven linears, one Hessian per input width) and prints its own line.

The JSON line also carries the roofline of the dominant kernel (the fused
SBA GEMM + KL kernel, timed live with HIP events on its own launch stream)
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_HBM_BPS = 8.0e12      # MI355X HBM3E
# fp32 vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one lane-op per cycle
PEAK_VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
# SQC's algorithmic ALU work per weight: 51 tau candidates x 9 float32 lane-ops
# (w*r, +z, round, clamp low, clamp high, -z, *s, w - w_hat, weighted square sum)
SQC_LANE_OPS_PER_PARAM = 51 * 9


def _dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


# Sources that make up the SBA GEMM + KL kernel: HBM traffic measured with
# counters is only reported while these are byte-identical to what was profiled.
SBA_SOURCES = ("post_mixed_precision_amd/csrc/sba.hip", "post_mixed_precision_amd/csrc/common.hpp",
               "post_mixed_precision_amd/csrc/kernels.hpp")


def sba_source_digest() -> str:
    """Digest of the kernel's code with comments and blank space removed."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in SBA_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, linear: str, group: int):
    """HBM bytes per launch of the SBA kernel from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE runs, scaled by a plain copy of known size), or
    None when there is no summary for this workload or the kernel has changed."""
    path = os.path.join(ROOT, "profiles", f"sba_klgemm.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "\t")):
            key, _, val = line.partition(":")
            kv[key.strip()] = val.strip()
    try:
        if (kv.get("source_digest") != sba_source_digest() or kv.get("linear") != linear
                or int(kv.get("group", -1)) != group):
            return None
        return {"fetch_bytes": float(kv["fetch_bytes_per_launch"]),
                "write_bytes": float(kv["write_bytes_per_launch"]),
                "copy_scale": float(kv["copy_scale"]), "source_digest": kv["source_digest"]}
    except (KeyError, ValueError):
        return None


def run_step(slim, X, W, group, N, ev=None, variant=None, gptq=False, lwc_iters=0):
    """One pass of the whole path; optional event list records stage boundaries."""
    def mark(i):
        if ev is not None:
            ev[i].record()
    mark(0)
    H = slim.hessian(X)
    mark(1)
    if gptq:   # the salience sweep also yields the factor GPTQ reads
        hinv, gsal, info, _, U = slim.salience(H, W, group, 0.01, want_u=True)
    else:
        hinv, gsal, info, _ = slim.salience(H, W, group, 0.01)
    mark(2)
    if variant is None:
        bits, kl, rs = slim.sba_search(X, W, gsal, group, N)
    else:   # ablation variant: objective and/or a given group order
        objective, order = variant
        bits, kl, rs = slim.sba_search_ex(X, W, group, N, group_sal=None if order is not None else gsal,
                                          order=order, objective=objective)
    mark(3)
    if gptq:   # the quantizer inside GPTQ's error-compensating sweep
        sq = slim.gptq_quantize(None, W, bits, hinv, group, 0.01, 0.1, 50, want_tau=False, U=U)
    elif lwc_iters:   # SliM-LLM+: learnable weight clipping in place of SQC
        sq = slim.lwc_calibrate(W, bits, H, X.shape[0], group, iters=lwc_iters)
        run_step.lwc_loss = sq["loss"]
    else:
        sq = slim.sqc_calibrate(W, bits, hinv, group, 0.1, 50, want_tau=False)
    mark(4)
    packed, pinfo = slim.pack(sq["codes"], bits, group, N)
    mark(5)
    run_step.last = (bits, packed, sq["scale"], sq["zero"])   # for the serving measurement
    return info, pinfo, rs, kl


def cpu_baseline(wl, lin_idx, group, N, Xh, Wh):
    """The oracle as it stands, on a bounded sample; stage costs scaled to the layer.

    Hessian: a token sample (cost linear in T).  Salience: full width (its
    inverse is O(m^3), its salience pass O(nm)).  SBA scan: a row sample of W,
    timed at two token counts; the fitted fixed + per-token cost is scaled to
    all tokens and to all rows (every step's work is linear in n).  SQC and
    packing: row samples (linear in n)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    lin = wl.linears[lin_idx]
    n, m, T = lin.n, lin.m, wl.tokens
    storage = wl.dtype
    k = m // group
    measured = 0.0
    t_h = min(T, 4096)
    t0 = time.perf_counter()
    H = oracle.hessian(Xh[:t_h])
    dt = time.perf_counter() - t0
    measured += dt
    s_hess = dt * T / t_h
    # salience needs a full-width H; the sample's H stands in (same cost)
    t0 = time.perf_counter()
    d32, S, info = oracle.salience(H, Wh, group, 0.01)
    s_sal = time.perf_counter() - t0
    measured += s_sal
    # SBA: every step's cost is linear in the rows; fit fixed + per-token cost
    n_s = min(n, max(256, n // 16))
    rows = np.linspace(0, n - 1, n_s).astype(np.int64)
    Ws = Wh[rows]
    tk = (min(T, 128), min(T, 512))
    secs = []
    for ts in tk:
        t0 = time.perf_counter()
        bits, _, _ = oracle.sba_search(Xh[:ts], Ws, S, N, group, storage)
        secs.append(time.perf_counter() - t0)
    measured += sum(secs)
    per_tok = max(secs[1] - secs[0], 0.0) / max(tk[1] - tk[0], 1)
    fixed = max(secs[0] - per_tok * tk[0], 0.0)
    s_sba = (fixed + per_tok * T) * n / n_s
    # SQC on a row sample
    r_q = min(n, 256)
    t0 = time.perf_counter()
    sq = oracle.sqc_calibrate(Wh, bits, d32, group, 0.1, 50, rows=np.arange(r_q))
    dt = time.perf_counter() - t0
    measured += dt
    s_sqc = dt * n / r_q
    r_p = min(n, max(256, n // 16))
    codes = np.zeros((r_p, m), dtype=np.uint8)
    part = sq["codes"][:r_p]
    codes[:len(part)] = part
    t0 = time.perf_counter()
    oracle.pack_bitplanes(codes, bits, group)
    dt = time.perf_counter() - t0
    measured += dt
    s_pack = dt * n / r_p
    total = s_hess + s_sal + s_sba + s_sqc + s_pack
    return {
        "value": n * m / 1e6 / total, "unit": "Mparams/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"Hessian on {t_h} of {T} tokens (x{T / t_h:g}); salience at full width {m}; SBA scan over all "
                   f"{k // 2 + 1} steps on {n_s} of {n} rows at {tk[0]} and {tk[1]} tokens, fixed + per-token cost "
                   f"fitted and scaled to {T} tokens and {n} rows; SQC on {r_q} rows (x{n / r_q:g}); "
                   f"packing on {r_p} rows (x{n / r_p:g})"),
        "seconds_extrapolated": {"hessian": s_hess, "salience": s_sal, "sba": s_sba, "sqc": s_sqc,
                                 "pack": s_pack, "total": total},
        "seconds_measured": round(measured, 2),
    }


def qlinear_time(slim, torch, xq, packed, bits, scale, zero, group, N, reps=50):
    """Seconds per slim.qlinear call, from the library's HIP events around its kernels."""
    for _ in range(5):
        slim.qlinear(xq, packed, bits, scale, zero, group, N)
    torch.cuda.synchronize()
    slim.timing_enable(True)
    slim.timing_reset()
    for _ in range(reps):
        slim.qlinear(xq, packed, bits, scale, zero, group, N)
    torch.cuda.synchronize()
    ms, calls = slim.timing_read("qlinear")
    slim.timing_enable(False)
    return ms / max(calls, 1) * 1e-3


def qlinear_bench(slim, torch, args):
    """The packed-plane linear layer alone on a synthetic N x M layer: random
    plane words (every bit pattern is a valid code), widths avg_bits + 1 on the
    first third of the groups and avg_bits - 1 on the last third, positive
    scales, zeros in [0, 2^bits)."""
    n, m = (int(v) for v in args.qlinear_shape.lower().split("x"))
    group = args.group or 128
    N = 2
    k = m // group
    bits = np.full(k, N, dtype=np.int8)
    bits[: k // 3] = N + 1
    bits[k - k // 3:] = N - 1
    rng = np.random.default_rng(7)
    words = n * m * N // 32
    packed = torch.from_numpy(rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
                              .view(np.int32)).to("cuda:0")
    bits_d = torch.from_numpy(bits).to("cuda:0")
    scale = torch.from_numpy(rng.uniform(1e-3, 2e-2, size=(n, k)).astype(np.float32)).to("cuda:0")
    zero = torch.from_numpy((rng.uniform(0, 1, size=(n, k)) * (2.0 ** bits[None, :] - 1)).astype(np.float32)).to("cuda:0")
    rep = {}
    for tq in (1, 8, 16, 64, 256, 1024, 2048):
        xq = torch.from_numpy(rng.standard_normal((tq, m)).astype(np.float32)).to("cuda:0").to(torch.bfloat16)
        sec = qlinear_time(slim, torch, xq, packed, bits_d, scale, zero, group, N, reps=50 if tq <= 256 else 10)
        qbytes = words * 4 + 2 * n * k * 4 + tq * m * 2 + tq * n * 4
        flops = 2.0 * tq * m * n
        # the binding roofline is the one whose ideal time is longer
        bound = "hbm" if qbytes / PEAK_HBM_BPS >= flops / PEAK_BF16_FLOPS else "mfma"
        rep[f"t{tq}"] = {"us_per_call": round(sec * 1e6, 2), "algorithmic_bytes": qbytes, "flops": flops,
                         "achieved_gbps": round(qbytes / sec / 1e9, 1),
                         "hbm_frac": round(qbytes / sec / PEAK_HBM_BPS, 4),
                         "achieved_tflops": round(flops / sec / 1e12, 2),
                         "mfma_frac": round(flops / sec / PEAK_BF16_FLOPS, 4), "bound": bound,
                         "frac": round(qbytes / sec / PEAK_HBM_BPS if bound == "hbm" else flops / sec / PEAK_BF16_FLOPS, 4)}
    out = {"metric": "packed-plane linear layer, GB/s of algorithmic bytes", "value": rep["t1"]["achieved_gbps"],
           "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"qlinear {n}x{m}", "n": n, "m": m, "group": group, "avg_bits": N},
           "roofline": {"bound": "hbm (t <= 64), mfma (prefill)", "kernel": "qlinear",
                        "peak_hbm_gbps": PEAK_HBM_BPS / 1e9, "peak_bf16_tflops": PEAK_BF16_FLOPS / 1e12, **rep}}
    print(json.dumps(out), flush=True)


def decoder_layer_bench(slim, torch, synth, args):
    """The whole 7B-shaped decoder layer: q/k/v/o 4096x4096, gate/up
    11008x4096, down 4096x11008, bf16; one calibration X per input width
    (262144 tokens each), so H is formed once per width and shared by the
    linears that read it, and so is diag(H_d^-1): the first linear of a width
    factors H, the others form their group means from its d.  A step is both
    Hessians and both factorisations plus salience, SBA, SQC and packing of
    all seven linears.  value = total params / 1e6 / seconds."""
    wl = synth.WORKLOADS["llama7b-decoder-layer"]
    group = args.group or 128
    N = wl.avg_bits
    Xd, Wd = {}, []
    for m in wl.widths:
        print(f"# generating X {wl.tokens}x{m}", file=sys.stderr, flush=True)
        Xd[m] = _dev(synth.make_x(wl, m), torch)
    for i, lin in enumerate(wl.linears):
        Wd.append(_dev(synth.make_w(wl, i), torch))
    torch.cuda.synchronize()

    def step(ev=None):
        H = {m: slim.hessian(X) for m, X in Xd.items()}
        if ev is not None:
            ev[1].record()
        infos = []
        hinv_w = {}
        for lin, W in zip(wl.linears, Wd):
            X = Xd[lin.m]
            if lin.m in hinv_w:
                hinv = hinv_w[lin.m]
                gsal, info, _ = slim.group_salience(hinv, W, group)
            else:
                hinv, gsal, info, _ = slim.salience(H[lin.m], W, group, 0.01)
                hinv_w[lin.m] = hinv
            bits, kl, rs = slim.sba_search(X, W, gsal, group, N)
            sq = slim.sqc_calibrate(W, bits, hinv, group, 0.1, 50, want_tau=False)
            packed, pinfo = slim.pack(sq["codes"], bits, group, N)
            infos.append((info, pinfo))
        return infos

    for i in range(args.warmup):
        infos = step()
        torch.cuda.synchronize()
        print(f"# warmup {i}", file=sys.stderr, flush=True)
    assert all(int(a.item()) == 0 and int(b.item()) == 0 for a, b in infos)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        evs[s_][0].record()
        step(evs[s_])
        evs[s_][2].record()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    h_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    params = sum(l.n * l.m for l in wl.linears)
    out = {"metric": "Mparams quantized/s per decoder layer (seven linears, one Hessian per input width)",
           "value": round(params / 1e6 / sec, 3), "unit": "Mparams/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 3), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; stands in for 128x2048 WikiText2 tokens and LLaMA weights)",
           "config": {"workload": "llama7b-decoder-layer", "linears": [f"{l.name} {l.n}x{l.m}" for l in wl.linears],
                      "tokens": wl.tokens, "group": group, "avg_bits": N, "hessians": len(Xd),
                      "factorisations": len(Xd)},
           "hessians_ms": round(h_ms, 3)}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="large-13b-70b")
    ap.add_argument("--linear", type=int, default=None,
                    help="index of the linear in the workload (default: the last, the largest of large-13b-70b)")
    ap.add_argument("--decoder-layer", action="store_true",
                    help="time the whole 7B-shaped decoder layer (seven linears, one Hessian per input width) "
                         "and print its own JSON line")
    ap.add_argument("--group", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--objective", choices=("kl", "mse"), default="kl",
                    help="SBA objective (the method's is kl; mse is the ablation)")
    ap.add_argument("--order", choices=("salience", "head_tail", "random"), default="salience",
                    help="group order of the SBA scan (the method's is salience)")
    ap.add_argument("--ablation-report", action="store_true",
                    help="also run the scan once per objective/order and report r* and the best score")
    ap.add_argument("--gptq", action="store_true",
                    help="calibrate and quantize the groups inside GPTQ's error-compensating sweep")
    ap.add_argument("--lwc", type=int, default=0, metavar="ITERS",
                    help="SliM-LLM+: calibrate with learnable weight clipping (ITERS Adam steps) in place of SQC")
    ap.add_argument("--qlinear-shape", default=None,
                    help="NxM: time only the packed-plane linear layer on a synthetic N x M layer "
                         "(random planes, widths avg_bits +- 1) and print its own JSON line")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the steps (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the quantizer runs one layer on one device here, and "
              "multi-GPU figures are not produced; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import post_mixed_precision_amd as slim
    if not os.path.exists(os.path.join(ROOT, "post_mixed_precision_amd", "libslim.so")):
        from post_mixed_precision_amd import build as _b
        _b.build()
    slim.load_library()

    if args.qlinear_shape:
        qlinear_bench(slim, torch, args)
        return

    if args.decoder_layer:
        decoder_layer_bench(slim, torch, synth, args)
        return

    wl = synth.WORKLOADS[args.workload]
    if args.linear is None:
        args.linear = len(wl.linears) - 1
    lin = wl.linears[args.linear]
    group = args.group or wl.groups[0]
    N = wl.avg_bits
    n, m, T = lin.n, lin.m, wl.tokens
    print(f"# generating {args.workload}/{lin.name}: W {n}x{m}, X {T}x{m} {wl.dtype}", file=sys.stderr, flush=True)
    Xh = synth.make_x(wl, m)
    Wh = synth.make_w(wl, args.linear)
    X, W = _dev(Xh, torch), _dev(Wh, torch)
    torch.cuda.synchronize()
    if args.copy_probe_mib > 0:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE in a counter
        # run calibrate the counters' units against bytes actually moved.
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy probe: {nbytes} bytes read and written", file=sys.stderr, flush=True)
        del src, dst

    k = m // group
    variant = None
    if args.objective != "kl" or args.order != "salience":
        if args.order == "salience":
            order = None
        else:
            perm = (np.arange(k) if args.order == "head_tail"
                    else np.random.default_rng([0, 0x5BA]).permutation(k))   # seeded random order
            order = torch.from_numpy(perm.astype(np.int32)).to("cuda:0")
        variant = (args.objective, order)

    for i in range(args.warmup):
        info, pinfo, rs, kl = run_step(slim, X, W, group, N, variant=variant, gptq=args.gptq, lwc_iters=args.lwc)
        torch.cuda.synchronize()
        print(f"# warmup {i}: info={int(info.item())} r*={int(rs.item())}", file=sys.stderr, flush=True)
    assert int(info.item()) == 0 and int(pinfo.item()) == 0

    # timed region: K whole steps, synchronised on both sides.  The library's
    # events go around the once-per-step kernels only; those launched per panel
    # or per group are timed in one extra step afterwards, outside the region.
    per_panel = ("chol_update", "gptq_sweep", "gptq_trail") + (("sqc_calibrate",) if args.gptq else ())
    slim.timing_enable(True)
    for nm in per_panel:
        slim.timing_select(nm, False)
    slim.timing_reset()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(slim, X, W, group, N, evs[s], variant=variant, gptq=args.gptq, lwc_iters=args.lwc)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    slim.timing_enable(False)
    sec = wall / args.steps
    names = ["hessian", "salience", "sba", "sqc", "pack"]
    stages = {nm: float(np.median([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
              for i, nm in enumerate(names)}
    kms, klaunch = slim.timing_read("sba_klgemm")
    ms_per_launch = kms / max(klaunch, 1)
    launches_per_step = klaunch / args.steps
    # algorithmic work of the scan: 6*T*m*n flops per layer (Y, Yhat_0 and every
    # group's one change of width), split evenly over the launches of a step
    flops_per_launch = 6.0 * T * m * n / launches_per_step
    achieved = flops_per_launch / (ms_per_launch * 1e-3)
    hms, hl = slim.timing_read("hessian_gram")
    lwc_ms, lwc_l = slim.timing_read("lwc_dh")
    qms, ql = slim.timing_read("sqc_calibrate")
    q_step = qms / args.steps
    pms, pl = slim.timing_read("pack_planes")
    # the per-panel and per-group kernels: one untimed step with only those
    slim.timing_enable(True)
    for nm in ("hessian_gram", "chol_update", "sba_klgemm", "sqc_calibrate", "pack_planes", "qlinear",
               "gptq_sweep", "gptq_trail"):
        slim.timing_select(nm, nm in per_panel)
    slim.timing_reset()
    run_step(slim, X, W, group, N, variant=variant, gptq=args.gptq, lwc_iters=args.lwc)
    torch.cuda.synchronize()
    slim.timing_enable(False)
    if args.gptq:
        q_step, ql = slim.timing_read("sqc_calibrate")
    cms, cl = slim.timing_read("chol_update")
    gsms, gsl = slim.timing_read("gptq_sweep")
    gtms, gtl = slim.timing_read("gptq_trail")
    print(f"# sba_klgemm {ms_per_launch:.3f} ms/launch ({launches_per_step:.0f}/step); "
          f"stages ms {json.dumps({k: round(v, 3) for k, v in stages.items()})}", file=sys.stderr, flush=True)

    value = n * m / 1e6 / sec
    out = {
        "metric": "Mparams quantized/s per linear layer; % of MFMA and HBM roofline",
        "value": round(value, 3), "unit": "Mparams/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; stands in for 128x2048 WikiText2 tokens and LLaMA weights)",
        "config": {"workload": args.workload, "linear": lin.name, "n": n, "m": m, "tokens": T,
                   "group": group, "avg_bits": N, "tau_lambda": wl.tau_lambda, "tau_steps": wl.tau_steps,
                   "sba_objective": args.objective, "sba_order": args.order,
                   "backbone": "gptq" if args.gptq else "none",
                   "calibration": f"lwc ({args.lwc} Adam steps)" if args.lwc else "sqc"},
        "roofline": {"bound": "mfma", "kernel": "sba_klgemm", "achieved": round(achieved / 1e12, 2),
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_FLOPS, 4), "traffic": None,
                     "ms_per_launch": round(ms_per_launch, 3), "algorithmic_flops_per_launch": flops_per_launch},
        "stages_ms": {k: round(v, 3) for k, v in stages.items()},
        "kernels_ms_per_step": {"sba_klgemm": round(kms / args.steps, 3),
                                "hessian_gram": round(hms / args.steps, 3),
                                "chol_update": round(cms, 3),
                                "sqc_calibrate": round(q_step, 3),
                                "pack_planes": round(pms / args.steps, 3)},
    }
    tr = measured_traffic(args.workload, lin.name, group)
    if tr is not None:
        out["roofline"]["traffic"] = round(tr["fetch_bytes"] + tr["write_bytes"])
        out["roofline"]["traffic_detail"] = {
            "unit": "bytes per launch", "fetch": round(tr["fetch_bytes"]), "write": round(tr["write_bytes"]),
            "copy_scale": tr["copy_scale"], "source_digest": tr["source_digest"],
            "algorithmic_bytes": 2 * (T * m + 4 * n * m) / launches_per_step}
    out["roofline"]["source_digest"] = sba_source_digest()
    from post_mixed_precision_amd import _lib as _slim_lib
    out["library_built_from_tree"] = _slim_lib.library_is_current()
    hess_flops = T * m * (m + 1)
    ro = out.setdefault("roofline_other", {})
    if hl:
        ro["hessian_gram"] = {"bound": "mfma", "achieved_tflops": round(hess_flops / (hms / hl * 1e-3) / 1e12, 2),
                              "frac": round(hess_flops / (hms / hl * 1e-3) / PEAK_BF16_FLOPS, 4)}
    if ql and q_step > 0:
        ro["sqc_calibrate"] = {
            "bound": "alu", "unit": "lane-op/s", "peak": PEAK_VALU_LANE_OPS,
            "lane_ops_per_param": SQC_LANE_OPS_PER_PARAM,
            "achieved": round(n * m * SQC_LANE_OPS_PER_PARAM / (q_step * 1e-3), -9),
            "frac": round(n * m * SQC_LANE_OPS_PER_PARAM / (q_step * 1e-3) / PEAK_VALU_LANE_OPS, 4),
            "hbm_gbps": round(n * m * (2 + 1 + 0.125) / (q_step * 1e-3) / 1e9, 1),
            "hbm_frac": round(n * m * (2 + 1 + 0.125) / (q_step * 1e-3) / PEAK_HBM_BPS, 4)}
    # salience: the float64 Cholesky sweep factors H_d (m^3/3 flops) and
    # inverts the factor alongside (another m^3/3), on the f64 matrix cores;
    # timed as the whole stage (its kernels run per panel)
    sal_ms = stages["salience"]
    if sal_ms > 0:
        f = 2.0 * m ** 3 / 3.0
        ro["salience"] = {"bound": "mfma", "dtype": "f64", "flops": f, "ms": round(sal_ms, 3),
                          "achieved_tflops": round(f / (sal_ms * 1e-3) / 1e12, 2), "peak": 78.6,
                          "frac": round(f / (sal_ms * 1e-3) / 78.6e12, 4),
                          "factor_only_frac": round(f / 2.0 / (sal_ms * 1e-3) / 78.6e12, 4)}
    if pl:
        ro["pack_planes"] = {"bound": "hbm", "bytes": n * m * (1 + N / 8),
                             "achieved_gbps": round(n * m * (1 + N / 8) / (pms / pl * 1e-3) / 1e9, 1),
                             "frac": round(n * m * (1 + N / 8) / (pms / pl * 1e-3) / PEAK_HBM_BPS, 4)}
    # The quantized layer served from its own planes (the deployment side):
    # Y = X W_hat^T for decode batches, timed per call with HIP events around
    # its kernels; outside the step's timed region.
    bits_l, packed_l, scale_l, zero_l = run_step.last
    qrep = {}
    for tq in (1, 8):
        xq = X[:tq].contiguous()
        sec_q = qlinear_time(slim, torch, xq, packed_l, bits_l, scale_l, zero_l, group, N)
        qbytes = packed_l.numel() * 4 + 2 * n * k * 4 + tq * m * xq.element_size() + tq * n * 4
        qrep[f"t{tq}"] = {"us_per_call": round(sec_q * 1e6, 2), "algorithmic_bytes": qbytes,
                          "achieved_gbps": round(qbytes / sec_q / 1e9, 1),
                          "frac": round(qbytes / sec_q / PEAK_HBM_BPS, 4)}
    out.setdefault("roofline_other", {})["qlinear"] = {"bound": "hbm", **qrep}
    if args.gptq:
        out["kernels_ms_per_step"]["gptq_sweep"] = round(gsms, 3)
        out["kernels_ms_per_step"]["gptq_trail"] = round(gtms, 3)
        # trailing products: sum over groups of 2 n g (m - (j+1) g) = n m (m - g) flops per step
        tflops = n * m * (m - group) / (gtms * 1e-3) / 1e12 if gtl else 0.0
        out.setdefault("roofline_other", {})["gptq_trail"] = {"bound": "mfma", "achieved_tflops": round(tflops, 2),
                                                              "peak": 78.6, "frac": round(tflops / 78.6, 4)}
    if args.lwc:
        lms, ll = lwc_ms, lwc_l
        f = 2.0 * n * m * m           # D H per iteration
        out["kernels_ms_per_step"]["lwc_dh"] = round(lms / args.steps, 3)
        if ll:
            out.setdefault("roofline_other", {})["lwc_dh"] = {
                "bound": "mfma", "dtype": "f64", "achieved_tflops": round(f / (lms / ll * 1e-3) / 1e12, 2),
                "peak": 78.6, "frac": round(f / (lms / ll * 1e-3) / 78.6e12, 4)}
        lo = run_step.lwc_loss.cpu().numpy()
        out["lwc_output_mse"] = {"start": float(lo[0]), "end": float(lo[-1]), "iters": args.lwc}
    if args.ablation_report:
        # The pages' ablation structure on this layer: the scan under each
        # objective and group order (untimed; r* and the best score).
        H = slim.hessian(X)
        _, gsal, _, _ = slim.salience(H, W, group, 0.01)
        rep = {}
        for obj in ("kl", "mse"):
            for ordk in ("salience", "head_tail", "random"):
                o = None if ordk == "salience" else torch.from_numpy(
                    (np.arange(k) if ordk == "head_tail" else np.random.default_rng([0, 0x5BA]).permutation(k))
                    .astype(np.int32)).to("cuda:0")
                b, sc, r = slim.sba_search_ex(X, W, group, N, group_sal=gsal if o is None else None, order=o,
                                              objective=obj)
                scn = sc.cpu().numpy()
                rep[f"{obj}/{ordk}"] = {"r_star": int(r.item()), "best": float(scn.min()), "r0": float(scn[0])}
        out["ablation"] = rep
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.linear, group, N, Xh, Wh)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
