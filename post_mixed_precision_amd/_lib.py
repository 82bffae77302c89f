"""ctypes binding of libslim.so (argument marshalling only).

Every computation runs in the HIP kernels behind include/slim.h; this module
only allocates outputs and workspaces with torch on the device, passes raw
pointers and the current HIP stream, and turns status codes into exceptions.
There is no fallback: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libslim.so")

SLIM_F32, SLIM_BF16 = 0, 1
STATUS = {0: "SLIM_OK", -1: "SLIM_E_NULL", -2: "SLIM_E_SHAPE", -3: "SLIM_E_DTYPE",
          -4: "SLIM_E_PARAM", -5: "SLIM_E_WORKSPACE", -6: "SLIM_E_HIP", -7: "SLIM_E_ALIGN"}

_c_i64, _c_int, _c_dbl, _c_vp, _c_sz = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t

_SIGS = {
    "slim_version": (_c_int, []),
    "slim_status_string": (ctypes.c_char_p, [_c_int]),
    "slim_last_hip_error": (_c_int, []),
    "slim_hessian_workspace": (_c_sz, [_c_i64, _c_i64, _c_int]),
    "slim_hessian": (_c_int, [_c_vp, _c_int, _c_i64, _c_i64, _c_vp, _c_int, _c_vp, _c_sz, _c_vp]),
    "slim_salience_workspace": (_c_sz, [_c_i64, _c_i64, _c_int]),
    "slim_salience": (_c_int, [_c_vp, _c_i64, _c_dbl, _c_vp, _c_int, _c_i64, _c_int, _c_vp, _c_vp, _c_vp,
                               _c_vp, _c_vp, _c_sz, _c_vp]),
    "slim_salience_u": (_c_int, [_c_vp, _c_i64, _c_dbl, _c_vp, _c_int, _c_i64, _c_int, _c_vp, _c_vp, _c_vp,
                                 _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "slim_group_salience_workspace": (_c_sz, [_c_i64, _c_i64, _c_int]),
    "slim_group_salience": (_c_int, [_c_vp, _c_i64, _c_vp, _c_int, _c_i64, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                     _c_sz, _c_vp]),
    "slim_sba_workspace": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_int, _c_int]),
    "slim_sba_search": (_c_int, [_c_vp, _c_int, _c_i64, _c_vp, _c_int, _c_i64, _c_i64, _c_int, _c_vp, _c_int,
                                 _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "slim_sba_search_ex": (_c_int, [_c_vp, _c_int, _c_i64, _c_vp, _c_int, _c_i64, _c_i64, _c_int, _c_vp, _c_vp,
                                    _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "slim_sqc_calibrate": (_c_int, [_c_vp, _c_int, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_dbl, _c_int, _c_vp,
                                    _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "slim_gptq_workspace": (_c_sz, [_c_i64, _c_i64, _c_int]),
    "slim_gptq_quantize": (_c_int, [_c_vp, _c_i64, _c_dbl, _c_vp, _c_int, _c_i64, _c_int, _c_vp, _c_vp, _c_dbl,
                                    _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "slim_gptq_quantize_u": (_c_int, [_c_vp, _c_i64, _c_vp, _c_int, _c_i64, _c_int, _c_vp, _c_vp, _c_dbl, _c_int,
                                      _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "slim_lwc_workspace": (_c_sz, [_c_i64, _c_i64, _c_int, _c_int]),
    "slim_lwc_calibrate": (_c_int, [_c_vp, _c_int, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_i64, _c_int, _c_dbl,
                                    _c_dbl, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "slim_tau_table": (_c_int, [_c_dbl, _c_int, _c_vp]),
    "slim_pack_words": (_c_i64, [_c_i64, _c_i64, _c_int]),
    "slim_pack": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_int, _c_vp, _c_vp, _c_vp]),
    "slim_qlinear_workspace": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_int]),
    "slim_qlinear": (_c_int, [_c_vp, _c_int, _c_i64, _c_i64, _c_vp, _c_vp, _c_int, _c_vp, _c_vp, _c_i64, _c_int,
                              _c_vp, _c_vp, _c_sz, _c_vp]),
    "slim_qlinear_noalloc_scratch_bytes": (_c_sz, []),
    "slim_qlinear_noalloc": (_c_int, [_c_vp, _c_int, _c_i64, _c_i64, _c_vp, _c_vp, _c_int, _c_vp, _c_vp, _c_i64,
                                      _c_int, _c_vp, _c_vp]),
    "slim_timing_enable": (_c_int, [_c_int]),
    "slim_timing_select": (_c_int, [ctypes.c_char_p, _c_int]),
    "slim_timing_reset": (_c_int, []),
    "slim_timing_read": (_c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_i64)]),
}

_lib = None


class SlimError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libslim.so (import torch first so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libslim.so not built at {path}; run post_mixed_precision_amd.build.build()")
    try:
        import torch  # noqa: F401  (loads torch's HIP runtime first: same soname, one runtime)
    except Exception:  # pragma: no cover
        pass
    _warn_if_stale(path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def library_is_current(path: str = LIB_PATH) -> bool:
    """True when the library was built from the sources now in the tree."""
    from . import build
    try:
        with open(path + ".sources") as f:
            return f.read().strip() == build.source_digest()
    except OSError:
        return False


def _warn_if_stale(path: str):
    if not library_is_current(path):
        import sys
        print(f"warning: {path} was not built from the current csrc/ and include/ sources; "
              "rebuild with post_mixed_precision_amd.build.build()", file=sys.stderr, flush=True)


def check(status: int, what: str):
    if status != 0:
        lib = load_library()
        msg = lib.slim_status_string(status).decode()
        extra = f" (hipError {lib.slim_last_hip_error()})" if status == -6 else ""
        raise SlimError(f"{what}: {STATUS.get(status, status)}: {msg}{extra}")


# --------------------------------------------------------------------------
# torch-facing wrappers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SLIM_BF16
    if t.dtype == torch.float32:
        return SLIM_F32
    raise SlimError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dev(t):
    torch = _torch()
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise SlimError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise SlimError("tensors must be contiguous")
    return t


def _arg(t, name: str, shape=None, dtypes=None, min_numel=None):
    """Check a tensor argument on the host before anything is launched: its
    dtype and its exact shape (None entries are free) or minimum element
    count.  The C ABI sees only pointers and the sizes passed beside them, so
    a tensor of the wrong size would become an out-of-bounds access on the
    device; this is where that is stopped.  Residency is checked afterwards,
    for all arguments at once (_on_gpu)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise SlimError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if dtypes is not None and t.dtype not in dtypes:
        raise SlimError(f"{name}: dtype {t.dtype}, expected one of {list(dtypes)}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and int(a) != int(s) for a, s in zip(t.shape, shape)):
            raise SlimError(f"{name}: shape {tuple(t.shape)}, expected {tuple('*' if s is None else s for s in shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise SlimError(f"{name}: {t.numel()} elements, at least {min_numel} needed")
    return t


def _on_gpu(*ts):
    """Every given tensor is contiguous, in GPU memory, on one device."""
    ts = [t for t in ts if t is not None]
    for t in ts:
        _dev(t)
    devs = {t.device for t in ts}
    if len(devs) > 1:
        raise SlimError(f"tensors live on different devices: {sorted(map(str, devs))}")


def _group_count(m: int, group: int) -> int:
    if group not in (32, 64, 128) or m % group != 0:
        raise SlimError(f"group {group} must be 32, 64 or 128 and divide m = {m}")
    return m // group


def _float_types():
    torch = _torch()
    return (torch.bfloat16, torch.float32)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _ws(nbytes: int, device):
    return _torch().empty(max(int(nbytes), 256), dtype=_torch().uint8, device=device)


def hessian(X, H=None, accumulate: bool = False):
    """H (+)= 2 X^T X, X [T, m] bf16/f32 on the GPU -> H float32 [m, m]."""
    torch = _torch()
    lib = load_library()
    X = _arg(X, "X", (None, None), _float_types())
    T, m = X.shape
    if H is None:
        if accumulate:
            raise SlimError("accumulate=True needs the H to add to")
        _on_gpu(X)
        H = torch.empty((m, m), dtype=torch.float32, device=X.device)
    else:
        H = _arg(H, "H", (m, m), (torch.float32,))
        _on_gpu(X, H)
    ws = _ws(lib.slim_hessian_workspace(T, m, _dtype_code(X)), X.device)
    check(lib.slim_hessian(_ptr(X), _dtype_code(X), T, m, _ptr(H), int(accumulate), _ptr(ws), ws.numel(),
                           _stream(X.device)), "slim_hessian")
    return H


def salience(H, W, group: int, damp_frac: float = 0.01, elem: bool = False, want_u: bool = False):
    """-> (hinv_diag f32 [m], group_sal f64 [k], info i32 [1], elem_sal f32 [n, m] or None), and with
    want_u the upper Cholesky factor U f64 [m, m] of H_d^-1 appended (slim_salience_u)."""
    torch = _torch()
    lib = load_library()
    W = _arg(W, "W", (None, None), _float_types())
    n, m = W.shape
    k = _group_count(m, group)
    H = _arg(H, "H", (m, m), (torch.float32,))
    _on_gpu(H, W)
    hinv = torch.empty(m, dtype=torch.float32, device=W.device)
    gsal = torch.empty(k, dtype=torch.float64, device=W.device)
    info = torch.zeros(1, dtype=torch.int32, device=W.device)
    esal = torch.empty((n, m), dtype=torch.float32, device=W.device) if elem else None
    ws = _ws(lib.slim_salience_workspace(n, m, group), W.device)
    if want_u:
        U = torch.empty((m, m), dtype=torch.float64, device=W.device)
        check(lib.slim_salience_u(_ptr(H), m, float(damp_frac), _ptr(W), _dtype_code(W), n, group, _ptr(hinv),
                                  _ptr(gsal), _ptr(esal), _ptr(U), _ptr(info), _ptr(ws), ws.numel(),
                                  _stream(W.device)), "slim_salience_u")
        return hinv, gsal, info, esal, U
    check(lib.slim_salience(_ptr(H), m, float(damp_frac), _ptr(W), _dtype_code(W), n, group, _ptr(hinv), _ptr(gsal),
                            _ptr(esal), _ptr(info), _ptr(ws), ws.numel(), _stream(W.device)), "slim_salience")
    return hinv, gsal, info, esal


def group_salience(hinv, W, group: int, elem: bool = False):
    """-> (group_sal f64 [k], info i32 [1], elem_sal f32 [n, m] or None) from a
    hinv_diag f32 [m] already formed (slim_group_salience): for the linears that
    share an input width, and so H, with the one that called salience()."""
    torch = _torch()
    lib = load_library()
    W = _arg(W, "W", (None, None), _float_types())
    n, m = W.shape
    k = _group_count(m, group)
    hinv = _arg(hinv, "hinv", (m,), (torch.float32,))
    _on_gpu(hinv, W)
    gsal = torch.empty(k, dtype=torch.float64, device=W.device)
    info = torch.zeros(1, dtype=torch.int32, device=W.device)
    esal = torch.empty((n, m), dtype=torch.float32, device=W.device) if elem else None
    ws = _ws(lib.slim_group_salience_workspace(n, m, group), W.device)
    check(lib.slim_group_salience(_ptr(hinv), m, _ptr(W), _dtype_code(W), n, group, _ptr(gsal), _ptr(esal),
                                  _ptr(info), _ptr(ws), ws.numel(), _stream(W.device)), "slim_group_salience")
    return gsal, info, esal


def sba_search(X, W, group_sal, group: int, avg_bits: int, ws_bytes: int | None = None):
    """-> (bits int8 [k], kl f64 [k//2+1], r_star int32 [1]).  ws_bytes: a
    workspace smaller than the preferred one makes the scan run its tokens
    in more batches (slim_sba_search's workspace rule)."""
    torch = _torch()
    lib = load_library()
    X = _arg(X, "X", (None, None), _float_types())
    T, m = X.shape
    W = _arg(W, "W", (None, m), _float_types())
    n = W.shape[0]
    k = _group_count(m, group)
    group_sal = _arg(group_sal, "group_sal", (k,), (torch.float64,))
    _on_gpu(X, W, group_sal)
    bits = torch.empty(k, dtype=torch.int8, device=W.device)
    kl = torch.empty(k // 2 + 1, dtype=torch.float64, device=W.device)
    rs = torch.empty(1, dtype=torch.int32, device=W.device)
    ws = _ws(lib.slim_sba_workspace(T, n, m, group, _dtype_code(W)) if ws_bytes is None else ws_bytes, W.device)
    check(lib.slim_sba_search(_ptr(X), _dtype_code(X), T, _ptr(W), _dtype_code(W), n, m, group, _ptr(group_sal),
                              int(avg_bits), _ptr(bits), _ptr(kl), _ptr(rs), _ptr(ws), ws.numel(),
                              _stream(W.device)), "slim_sba_search")
    return bits, kl, rs


OBJECTIVES = {"kl": 0, "mse": 1}


def sba_search_ex(X, W, group: int, avg_bits: int, group_sal=None, order=None, objective: str = "kl"):
    """Ablation variants: objective "kl" or "mse"; order (int32 [k] on the GPU)
    replaces the salience ranking.  -> (bits int8 [k], score f64 [k//2+1], r_star int32 [1])."""
    torch = _torch()
    lib = load_library()
    X = _arg(X, "X", (None, None), _float_types())
    T, m = X.shape
    W = _arg(W, "W", (None, m), _float_types())
    k = _group_count(m, group)
    if group_sal is None and order is None:
        raise SlimError("give group_sal (salience ranking) or order")
    if group_sal is not None:
        group_sal = _arg(group_sal, "group_sal", (k,), (torch.float64,))
    if order is not None:
        order = _arg(order, "order", (k,), (torch.int32,))
        # a permutation of the groups, checked on the host (k <= a few hundred)
        if sorted(order.cpu().tolist()) != list(range(k)):
            raise SlimError("order must be a permutation of 0..k-1")
    if objective not in OBJECTIVES:
        raise SlimError(f"unknown objective {objective!r}")
    _on_gpu(X, W, group_sal, order)
    n = W.shape[0]
    bits = torch.empty(k, dtype=torch.int8, device=W.device)
    score = torch.empty(k // 2 + 1, dtype=torch.float64, device=W.device)
    rs = torch.empty(1, dtype=torch.int32, device=W.device)
    ws = _ws(lib.slim_sba_workspace(T, n, m, group, _dtype_code(W)), W.device)
    check(lib.slim_sba_search_ex(_ptr(X), _dtype_code(X), T, _ptr(W), _dtype_code(W), n, m, group, _ptr(group_sal),
                                 _ptr(order), int(avg_bits), OBJECTIVES[objective], _ptr(bits), _ptr(score), _ptr(rs),
                                 _ptr(ws), ws.numel(), _stream(W.device)), "slim_sba_search_ex")
    return bits, score, rs


def sqc_calibrate(W, bits, hinv, group: int, lam: float = 0.1, n_tau: int = 50, want_tau: bool = True):
    """-> dict(scale, zero [n, k] f32; codes [n, m] u8; mask [n, m/32] i32 bits; tau_idx [n, k] u8)."""
    torch = _torch()
    lib = load_library()
    W = _arg(W, "W", (None, None), _float_types())
    n, m = W.shape
    k = _group_count(m, group)
    bits = _arg(bits, "bits", (k,), (torch.int8,))
    hinv = _arg(hinv, "hinv", (m,), (torch.float32,))
    _on_gpu(W, bits, hinv)
    dev = W.device
    out = {
        "scale": torch.empty((n, k), dtype=torch.float32, device=dev),
        "zero": torch.empty((n, k), dtype=torch.float32, device=dev),
        "codes": torch.empty((n, m), dtype=torch.uint8, device=dev),
        "mask": torch.empty((n, max(m // 32, 1)), dtype=torch.int32, device=dev),
        "tau_idx": torch.empty((n, k), dtype=torch.uint8, device=dev) if want_tau else None,
    }
    check(lib.slim_sqc_calibrate(_ptr(W), _dtype_code(W), n, m, group, _ptr(bits), _ptr(hinv), float(lam),
                                 int(n_tau), _ptr(out["scale"]), _ptr(out["zero"]), _ptr(out["codes"]),
                                 _ptr(out["mask"]), _ptr(out["tau_idx"]), _stream(dev)), "slim_sqc_calibrate")
    return out


def gptq_quantize(H, W, bits, hinv, group: int, damp_frac: float = 0.01, lam: float = 0.1, n_tau: int = 50,
                  want_tau: bool = True, U=None):
    """GPTQ sweep with the group quantizer -> dict(scale, zero [n, k] f32; codes [n, m] u8;
    mask [n, m/32] i32 bits; tau_idx [n, k] u8; info i32 [1]).  With U (the factor
    salience(..., want_u=True) returns) H may be None and is not factored again
    (slim_gptq_quantize_u)."""
    torch = _torch()
    lib = load_library()
    W = _arg(W, "W", (None, None), _float_types())
    n, m = W.shape
    k = _group_count(m, group)
    bits = _arg(bits, "bits", (k,), (torch.int8,))
    hinv = _arg(hinv, "hinv", (m,), (torch.float32,))
    if U is not None:
        U = _arg(U, "U", (m, m), (torch.float64,))
    else:
        if H is None:
            raise SlimError("give H, or the factor U")
        H = _arg(H, "H", (m, m), (torch.float32,))
    _on_gpu(W, bits, hinv, U, H)
    dev = W.device
    out = {
        "scale": torch.empty((n, k), dtype=torch.float32, device=dev),
        "zero": torch.empty((n, k), dtype=torch.float32, device=dev),
        "codes": torch.empty((n, m), dtype=torch.uint8, device=dev),
        "mask": torch.empty((n, max(m // 32, 1)), dtype=torch.int32, device=dev),
        "tau_idx": torch.empty((n, k), dtype=torch.uint8, device=dev) if want_tau else None,
        "info": torch.zeros(1, dtype=torch.int32, device=dev),
    }
    ws = _ws(lib.slim_gptq_workspace(n, m, group), dev)
    if U is not None:
        check(lib.slim_gptq_quantize_u(_ptr(U), m, _ptr(W), _dtype_code(W), n, group, _ptr(bits), _ptr(hinv),
                                       float(lam), int(n_tau), _ptr(out["scale"]), _ptr(out["zero"]),
                                       _ptr(out["codes"]), _ptr(out["mask"]), _ptr(out["tau_idx"]),
                                       _ptr(out["info"]), _ptr(ws), ws.numel(), _stream(dev)), "slim_gptq_quantize_u")
        return out
    check(lib.slim_gptq_quantize(_ptr(H), m, float(damp_frac), _ptr(W), _dtype_code(W), n, group, _ptr(bits),
                                 _ptr(hinv), float(lam), int(n_tau), _ptr(out["scale"]), _ptr(out["zero"]),
                                 _ptr(out["codes"]), _ptr(out["mask"]), _ptr(out["tau_idx"]), _ptr(out["info"]),
                                 _ptr(ws), ws.numel(), _stream(dev)), "slim_gptq_quantize")
    return out


def lwc_calibrate(W, bits, H, tokens: int, group: int, iters: int = 20, lr: float = 1e-2, init: float = 4.0,
                  want_logits: bool = False):
    """SliM-LLM+ learnable weight clipping -> dict(scale, zero [n, k] f32; codes [n, m] u8;
    loss f64 [iters+1]; logits f64 [2, n, k] or None).  H: the float32 Hessian of the
    `tokens` calibration tokens (slim.hessian)."""
    torch = _torch()
    lib = load_library()
    W = _arg(W, "W", (None, None), _float_types())
    n, m = W.shape
    k = _group_count(m, group)
    bits = _arg(bits, "bits", (k,), (torch.int8,))
    H = _arg(H, "H", (m, m), (torch.float32,))
    _on_gpu(W, bits, H)
    dev = W.device
    out = {
        "scale": torch.empty((n, k), dtype=torch.float32, device=dev),
        "zero": torch.empty((n, k), dtype=torch.float32, device=dev),
        "codes": torch.empty((n, m), dtype=torch.uint8, device=dev),
        "loss": torch.empty(iters + 1, dtype=torch.float64, device=dev),
        "logits": torch.empty((2, n, k), dtype=torch.float64, device=dev) if want_logits else None,
    }
    ws = _ws(lib.slim_lwc_workspace(n, m, group, iters), dev)
    check(lib.slim_lwc_calibrate(_ptr(W), _dtype_code(W), n, m, group, _ptr(bits), _ptr(H), int(tokens), int(iters),
                                 float(lr), float(init), _ptr(out["scale"]), _ptr(out["zero"]), _ptr(out["codes"]),
                                 _ptr(out["logits"]), _ptr(out["loss"]), _ptr(ws), ws.numel(), _stream(dev)),
          "slim_lwc_calibrate")
    return out


def pack(codes, bits, group: int, avg_bits: int):
    """-> (packed int32 words [n*m*N/32] (uint32 bit patterns), info int32 [1])."""
    torch = _torch()
    lib = load_library()
    codes = _arg(codes, "codes", (None, None), (torch.uint8,))
    n, m = codes.shape
    k = _group_count(m, group)
    bits = _arg(bits, "bits", (k,), (torch.int8,))
    _on_gpu(codes, bits)
    words = lib.slim_pack_words(n, m, avg_bits)
    if words < 0:
        raise SlimError("bad pack shape")
    packed = torch.zeros(max(words, 1), dtype=torch.int32, device=codes.device)
    info = torch.zeros(1, dtype=torch.int32, device=codes.device)
    check(lib.slim_pack(_ptr(codes), n, m, group, _ptr(bits), int(avg_bits), _ptr(packed), _ptr(info),
                        _stream(codes.device)), "slim_pack")
    return packed[:words], info


def qlinear(X, packed, bits, scale, zero, group: int, avg_bits: int):
    """Y = X W_hat^T from the packed planes: X [t, m] bf16/f32 (decode batches or prefill,
    t <= 65536) -> Y float32 [t, n]."""
    torch = _torch()
    lib = load_library()
    X = _arg(X, "X", (None, None), _float_types())
    T, m = X.shape
    k = _group_count(m, group)
    scale = _arg(scale, "scale", (None, k), (torch.float32,))
    n = scale.shape[0]
    zero = _arg(zero, "zero", (n, k), (torch.float32,))
    bits = _arg(bits, "bits", (k,), (torch.int8,))
    words = lib.slim_pack_words(n, m, avg_bits)
    if words < 0:
        raise SlimError("bad layer shape or average width")
    packed = _arg(packed, "packed", (None,), (torch.int32,), min_numel=words)
    _on_gpu(X, packed, bits, scale, zero)
    Y = torch.empty((T, n), dtype=torch.float32, device=X.device)
    ws = _ws(lib.slim_qlinear_workspace(T, n, m, group), X.device)
    check(lib.slim_qlinear(_ptr(X), _dtype_code(X), T, m, _ptr(packed), _ptr(bits), int(avg_bits), _ptr(scale),
                           _ptr(zero), n, group, _ptr(Y), _ptr(ws), ws.numel(), _stream(X.device)), "slim_qlinear")
    return Y


def qlinear_noalloc(X, packed, bits, scale, zero, group: int, avg_bits: int, Y=None):
    """slim_qlinear_noalloc: as qlinear, with the partial sums in the library's
    fixed device scratch instead of a workspace.  Y (float32 [t, n] on the
    GPU) may be given; then nothing at all is allocated for the call."""
    torch = _torch()
    lib = load_library()
    X = _arg(X, "X", (None, None), _float_types())
    T, m = X.shape
    k = _group_count(m, group)
    scale = _arg(scale, "scale", (None, k), (torch.float32,))
    n = scale.shape[0]
    zero = _arg(zero, "zero", (n, k), (torch.float32,))
    bits = _arg(bits, "bits", (k,), (torch.int8,))
    words = lib.slim_pack_words(n, m, avg_bits)
    if words < 0:
        raise SlimError("bad layer shape or average width")
    packed = _arg(packed, "packed", (None,), (torch.int32,), min_numel=words)
    if Y is not None:
        Y = _arg(Y, "Y", (T, n), (torch.float32,))
    _on_gpu(X, packed, bits, scale, zero, Y)
    if Y is None:
        Y = torch.empty((T, n), dtype=torch.float32, device=X.device)
    check(lib.slim_qlinear_noalloc(_ptr(X), _dtype_code(X), T, m, _ptr(packed), _ptr(bits), int(avg_bits),
                                   _ptr(scale), _ptr(zero), n, group, _ptr(Y), _stream(X.device)),
          "slim_qlinear_noalloc")
    return Y


def tau_table(lam: float = 0.1, n_tau: int = 50) -> np.ndarray:
    lib = load_library()
    out = np.zeros(n_tau + 1, dtype=np.float32)
    check(lib.slim_tau_table(float(lam), int(n_tau), out.ctypes.data_as(ctypes.c_void_p)), "slim_tau_table")
    return out


def timing_enable(on: bool = True):
    load_library().slim_timing_enable(int(on))


def timing_select(kernel: str, on: bool):
    """Leave one timed kernel out of (on=False) or back in the enabled timing."""
    check(load_library().slim_timing_select(kernel.encode(), int(on)), "slim_timing_select")


def timing_reset():
    load_library().slim_timing_reset()


def timing_read(kernel: str):
    """-> (total_ms, launches) for a timed kernel since the last reset."""
    lib = load_library()
    ms, cnt = ctypes.c_double(), _c_i64()
    check(lib.slim_timing_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(cnt)), "slim_timing_read")
    return ms.value, cnt.value
