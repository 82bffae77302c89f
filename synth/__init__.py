"""Seeded synthetic layers for the SliM-LLM per-layer quantizer path.

This module only draws random numbers, lays out outlier channels and stores
the drawn values in the layer's storage dtype (float32 -> bfloat16 with
round-to-nearest-even).  It holds none of the quantizer's arithmetic: the HIP
path's tests and benchmark and the CPU oracle both take their inputs from
here, and neither side's results ever flow back into it.

Shapes and structure follow the workloads the SliM-LLM pages describe
("SliM-LLM: Salience-Driven Mixed-Precision Quantization for Large Language
Models", blog digest on rkmt.cn, sections on the evaluation protocol and the
core design): calibration of 128 sequences x 2048 tokens, groups of 128 input
columns, LLaMA-shaped projections, and salient input channels that cluster
because activation channels carry outliers (its Theorem 1 and Fig. 3, which
place the clusters of LLaMA-7B layer 2 near channels 2100, 3218 and 3853).
No dataset or trained weights are used: WikiText2 calibration text and LLaMA
checkpoints are stood in for by these draws.

Every tensor has its own counter-keyed stream, ``numpy.random.default_rng``
seeded with ``[seed, workload id, tensor kind, ...]``.  Activations are drawn
per 2048-token chunk from a stream keyed by the chunk index, so any token
range can be regenerated on its own.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK_TOKENS = 2048            # one calibration sequence
CLUSTER_CENTRES_4096 = (2100, 3218, 3853)   # salient-channel clusters, width 4096

_KIND_LAYOUT, _KIND_X, _KIND_W = 0, 1, 2


# --------------------------------------------------------------------------
# storage conversion (not method arithmetic: how the drawn layer is stored)
# --------------------------------------------------------------------------
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.

    Inputs drawn here are finite, so no NaN handling is needed."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Linear:
    name: str
    n: int                      # output features (rows of W)
    m: int                      # input features (columns of W)
    dist: str                   # "normal" or "t5"
    std: float                  # scale of the draw


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                    # stream key
    tokens: int                 # calibration tokens T
    dtype: str                  # "bf16" or "f32"
    linears: tuple
    groups: tuple = (128,)      # group sizes to run
    avg_bits: int = 2
    tau_lambda: float = 0.1
    tau_steps: int = 50
    outlier_frac: float = 0.01  # fraction of input channels that are outliers
    outlier_scale: tuple = (10.0, 50.0)   # per-channel scale ~ U(lo, hi)
    tiny_bands: tuple = field(default=())  # explicit (count, scale) bands for the tiny layer

    @property
    def widths(self):
        out = []
        for lin in self.linears:
            if lin.m not in out:
                out.append(lin.m)
        return out


_Q = lambda name, n, m, dist, std: Linear(name, n, m, dist, std)   # noqa: E731

WORKLOADS = {
    "tiny-512": Workload(
        "tiny-512", 1, 2048, "f32", (_Q("w", 512, 512, "normal", 0.02),),
        tiny_bands=((8, 20.0), (8, 20.0))),
    "llama7b-attn-4096": Workload(
        "llama7b-attn-4096", 2, 262144, "bf16", (_Q("q_proj", 4096, 4096, "normal", 0.02),)),
    "llama7b-mlp-pair": Workload(
        "llama7b-mlp-pair", 3, 262144, "bf16",
        (_Q("up_proj", 11008, 4096, "t5", 0.02), _Q("down_proj", 4096, 11008, "t5", 0.02)),
        avg_bits=3),
    "llama7b-decoder-layer": Workload(
        "llama7b-decoder-layer", 4, 262144, "bf16",
        (_Q("q_proj", 4096, 4096, "normal", 0.02), _Q("k_proj", 4096, 4096, "normal", 0.02),
         _Q("v_proj", 4096, 4096, "normal", 0.02), _Q("o_proj", 4096, 4096, "normal", 0.02),
         _Q("gate_proj", 11008, 4096, "t5", 0.02), _Q("up_proj", 11008, 4096, "t5", 0.02),
         _Q("down_proj", 4096, 11008, "t5", 0.02)),
        groups=(128, 64, 32)),
    "large-13b-70b": Workload(
        "large-13b-70b", 5, 262144, "bf16",
        (_Q("mlp13b", 13824, 5120, "normal", 0.015), _Q("mlp70b", 28672, 8192, "normal", 0.015))),
}


def custom(name="custom", tokens=256, dtype="bf16", n=64, m=256, dist="normal", std=0.02,
           avg_bits=2, wid=99, outlier_frac=0.01):
    """A small workload of arbitrary shape with the same draw laws (for ragged cases)."""
    return Workload(name, wid, tokens, dtype, (_Q("w", n, m, dist, std),), avg_bits=avg_bits,
                    outlier_frac=outlier_frac)


# --------------------------------------------------------------------------
# outlier-channel layout
# --------------------------------------------------------------------------
def _run_lengths(total: int, runs: int):
    base, extra = divmod(total, runs)
    return [base + (1 if i < extra else 0) for i in range(runs)]


def outlier_layout(wl: Workload, m: int, seed: int = 0):
    """(channel indices int64, scales float32) of the outlier input channels.

    Runs are centred at round(p * m / 4096) for p in the three cluster
    positions; the tiny layer uses its explicit bands at the first two."""
    rng = np.random.default_rng([seed, wl.wid, _KIND_LAYOUT, m])
    chans, scales = [], []
    if wl.tiny_bands:
        for (count, scale), p in zip(wl.tiny_bands, CLUSTER_CENTRES_4096):
            c = int(np.floor(p * m / 4096 + 0.5))
            lo = c - count // 2
            chans.extend(range(lo, lo + count))
            scales.extend([scale] * count)
    else:
        total = int(round(wl.outlier_frac * m))
        if total > 0:
            for L, p in zip(_run_lengths(total, 3), CLUSTER_CENTRES_4096):
                c = int(np.floor(p * m / 4096 + 0.5))
                lo = max(0, min(m - L, c - L // 2))
                chans.extend(range(lo, lo + L))
        lo_s, hi_s = wl.outlier_scale
        scales = list(rng.uniform(lo_s, hi_s, size=len(chans)))
    ch = np.asarray(chans, dtype=np.int64)
    ch, idx = np.unique(ch, return_index=True)
    sc = np.asarray(scales, dtype=np.float32)[idx] if len(scales) else np.zeros(0, np.float32)
    keep = ch < m
    return ch[keep], sc[keep]


# --------------------------------------------------------------------------
# activations and weights
# --------------------------------------------------------------------------
def _x_chunk(wl: Workload, m: int, c: int, ch, sc, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, wl.wid, _KIND_X, m, c])
    a = rng.standard_normal((CHUNK_TOKENS, m), dtype=np.float32)
    if len(ch):
        a[:, ch] *= sc[None, :]
    return a


def make_x(wl: Workload, m: int, t0: int = 0, t1: int | None = None, seed: int = 0,
           threads: int | None = None) -> np.ndarray:
    """Calibration activations X[t0:t1, :m], token-major.

    Returns uint16 bfloat16 bits for a bf16 workload, float32 otherwise."""
    t1 = wl.tokens if t1 is None else t1
    assert 0 <= t0 <= t1
    ch, sc = outlier_layout(wl, m, seed)
    bf = wl.dtype == "bf16"
    out = np.empty((t1 - t0, m), dtype=np.uint16 if bf else np.float32)
    c0, c1 = t0 // CHUNK_TOKENS, (t1 + CHUNK_TOKENS - 1) // CHUNK_TOKENS

    def work(c):
        a = _x_chunk(wl, m, c, ch, sc, seed)
        lo, hi = max(t0, c * CHUNK_TOKENS), min(t1, (c + 1) * CHUNK_TOKENS)
        part = a[lo - c * CHUNK_TOKENS: hi - c * CHUNK_TOKENS]
        out[lo - t0: hi - t0] = to_bf16_bits(part) if bf else part

    threads = threads or min(16, os.cpu_count() or 1)
    if c1 - c0 <= 1:
        for c in range(c0, c1):
            work(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(c0, c1)))
    return out


def make_w(wl: Workload, index: int, seed: int = 0, threads: int | None = None) -> np.ndarray:
    """Weight of linear ``index``, [n, m] row-major (uint16 bf16 bits or float32)."""
    lin = wl.linears[index]
    bf = wl.dtype == "bf16"
    out = np.empty((lin.n, lin.m), dtype=np.uint16 if bf else np.float32)
    rows = 1024
    blocks = list(range(0, lin.n, rows))

    def work(bi):
        r0 = blocks[bi]
        r1 = min(lin.n, r0 + rows)
        rng = np.random.default_rng([seed, wl.wid, _KIND_W, index, bi])
        if lin.dist == "normal":
            a = rng.standard_normal((r1 - r0, lin.m), dtype=np.float32) * np.float32(lin.std)
        elif lin.dist == "t5":
            a = (rng.standard_t(5, size=(r1 - r0, lin.m)) * lin.std).astype(np.float32)
        else:
            raise ValueError(lin.dist)
        out[r0:r1] = to_bf16_bits(a) if bf else a

    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(len(blocks))))
    return out


def as_float(a: np.ndarray) -> np.ndarray:
    """Stored tensor -> float32 values (bf16 bits are widened exactly)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)
