"""One linear layer through the whole path, enqueued on the current stream.

Stage order as in the SliM-LLM blog digest (rkmt.cn), core design: Hessian
from calibration activations, salience, SBA bit allocation, SQC calibration,
then group-structured storage.  Nothing is copied back to the host between
stages; the caller synchronises once and may inspect ``info``.
"""
from __future__ import annotations

from . import _lib


def quantize_layer(X, W, group: int = 128, avg_bits: int = 2, lam: float = 0.1, n_tau: int = 50,
                   damp_frac: float = 0.01, H=None, gptq: bool = False, hinv=None):
    """X [T, m], W [n, m] (bf16 or f32, GPU).  If H is given the Hessian stage is
    skipped (a Hessian shared by several linears of one input width); if hinv,
    that H's diag((H + a I)^-1) from an earlier call, is given too, the
    factorisation is skipped as well and only the group means are formed.
    With gptq set, the groups are calibrated and quantized inside GPTQ's
    error-compensating sweep (the backbone the digest names) instead of
    independently (it reads the factor, so hinv is not taken then)."""
    if hinv is not None and (H is None or gptq):
        raise _lib.SlimError("hinv is taken with the H it came from, and not with gptq")
    if H is None:
        H = _lib.hessian(X)
    if gptq:   # the salience sweep also yields the factor GPTQ reads
        hinv, gsal, info, _, U = _lib.salience(H, W, group, damp_frac, want_u=True)
    elif hinv is not None:
        gsal, info, _ = _lib.group_salience(hinv, W, group)
    else:
        hinv, gsal, info, _ = _lib.salience(H, W, group, damp_frac)
    bits, kl, r_star = _lib.sba_search(X, W, gsal, group, avg_bits)
    if gptq:
        sq = _lib.gptq_quantize(None, W, bits, hinv, group, damp_frac, lam, n_tau, U=U)
        sq["gptq_info"] = sq.pop("info")
    else:
        sq = _lib.sqc_calibrate(W, bits, hinv, group, lam, n_tau)
    packed, pinfo = _lib.pack(sq["codes"], bits, group, avg_bits)
    return {"H": H, "hinv": hinv, "group_sal": gsal, "info": info, "bits": bits, "kl": kl, "r_star": r_star,
            "pack_info": pinfo, "packed": packed, **sq}
