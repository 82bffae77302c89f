"""The whole per-layer path, stage by stage.  TEST INFRASTRUCTURE (oracle).

Order as on page 1, "核心设计" (core design): Hessian from calibration
activations -> element and group salience -> SBA bit allocation -> SQC
calibration of each group's shared quantizer -> group-structured storage.
GPTQ's error compensation is not part of this path.
"""
from .hessian import hessian
from .salience import salience
from .sba import sba_search
from .sqc import sqc_calibrate
from .pack import pack_bitplanes


def quantize_layer(X, W, group: int = 128, avg_bits: int = 2, lam: float = 0.1,
                   n_tau: int = 50, damp_frac: float = 0.01, storage: str = "bf16"):
    H = hessian(X)
    d32, S, info = salience(H, W, group, damp_frac)
    if info != 0:
        return {"H": H, "info": info}
    bits, kl, r_star = sba_search(X, W, S, avg_bits, group, storage)
    sq = sqc_calibrate(W, bits, d32, group, lam, n_tau)
    packed = pack_bitplanes(sq["codes"], bits, group)
    return {"H": H, "d": d32, "S": S, "info": 0, "bits": bits, "kl": kl,
            "r_star": r_star, "sqc": sq, "packed": packed}
