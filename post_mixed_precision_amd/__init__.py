"""SliM-LLM per-layer quantizer path for MI355X (gfx950).

Five stages, each one C-ABI call into libslim.so (include/slim.h) running
hand-written HIP kernels:

    hessian        H = 2 X^T X                                  (MFMA bf16/f32)
    salience       d = diag((H + a I)^-1), group-mean w^2/d^2   (fp64 MFMA Cholesky)
    sba_search     balanced N-1/N/N+1 allocation scored by output KL (fused MFMA + softmax)
                   (sba_search_ex: output-MSE objective or a given group order, for the ablations)
    sqc_calibrate  3-sigma mask + tau grid over scale and zero  (wave-level, VALU)
                   (gptq_quantize: the same quantizer inside GPTQ's error-compensating sweep;
                    lwc_calibrate: SliM-LLM+, learnable weight clipping in its place)
    pack           group-structured bit-planes                  (HBM)
    qlinear        Y = X W_hat^T read from the planes (decode-sized batches)
                   (qlinear_noalloc: the same with no workspace, for callers that cannot allocate)

``quantize_layer`` chains them on the current stream.  PyTorch only provides
device memory and the stream.
"""
from ._lib import (SlimError, load_library, hessian, salience, group_salience, sba_search, sba_search_ex, sqc_calibrate, gptq_quantize,
                   lwc_calibrate, pack, qlinear, qlinear_noalloc, tau_table,
                   timing_enable, timing_select, timing_reset, timing_read, SLIM_F32, SLIM_BF16)
from .layer import quantize_layer

__all__ = ["SlimError", "load_library", "hessian", "salience", "group_salience", "sba_search", "sba_search_ex", "sqc_calibrate",
           "gptq_quantize", "lwc_calibrate", "pack", "qlinear", "qlinear_noalloc", "tau_table", "timing_enable", "timing_select", "timing_reset", "timing_read", "quantize_layer", "SLIM_F32",
           "SLIM_BF16"]
