"""CPU oracle for the SliM-LLM per-layer quantizer path.  TEST INFRASTRUCTURE.

This package is the slow, plainly written reference that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product package
(``post_mixed_precision_amd``) never does, and shares no code, table or
helper with it.

Source pages (cited by title and section throughout):

* "SliM-LLM: Salience-Driven Mixed-Precision Quantization for Large Language
  Models" -- the Chinese blog digest on rkmt.cn ("page 1"), section
  "核心设计" (core design): component one SBA (element salience, KL objective,
  the balance constraint, the double-pointer search over [0, k/2]) and
  component two SQC (the 3-sigma mask and the tau scaling of the shared
  quantizer over [1-lambda, 1+lambda], lambda = 0.1, n = 50); sections on the
  evaluation protocol (group 128, 128 x 2048 calibration tokens) and the FAQ
  (no bitmap, zero extra storage).
* The scime.ai summary page ("page 2"), section "Approach": bit-widths by
  average group salience, a KL-optimal ratio with balanced counts, scale and
  zero calibrated by a search over a clipping factor tau.

Precision: fp64 unless a step defines an integer decision in the kernel's
precision; the quantizer itself is a fixed float32 operation sequence so that
codes are comparable bit for bit.  Every reading of a point the pages leave
open is stated in the docstring of the function that takes it.

Pins (tests under ``tests/test_oracle_*.py``) tie every function here to
something other than itself: brute-force loops, closed forms, library
routines and the invariants the pages state.
"""
from .decode import as_f64, as_f32, bf16_round
from .hessian import hessian, hessian_entries
from .salience import hinv_diag, element_salience, group_salience, salience
from .quantizer import tau_grid, minmax_params, fake_quant, quant_codes
from .sba import (rank_groups, allocation, trial_weights, kl_divergence, output_mse, head_tail_order, random_order,
                  sba_search)
from .sqc import mask_3sigma, sqc_calibrate
from .pack import pack_bitplanes, unpack_bitplanes, packed_words
from .qlinear import dequant_weights, qlinear
from .gptq import upper_chol_inverse, gptq_quantize
from .lwc import lwc_calibrate
from .pipeline import quantize_layer

__all__ = [
    "as_f64", "as_f32", "bf16_round", "hessian", "hessian_entries", "hinv_diag",
    "element_salience", "group_salience", "salience", "tau_grid", "minmax_params",
    "fake_quant", "quant_codes", "rank_groups", "allocation", "trial_weights",
    "kl_divergence", "sba_search", "mask_3sigma", "sqc_calibrate", "pack_bitplanes",
    "unpack_bitplanes", "packed_words", "quantize_layer", "dequant_weights", "qlinear",
    "upper_chol_inverse", "gptq_quantize", "lwc_calibrate",
]
