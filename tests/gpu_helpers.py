"""Helpers shared by the GPU parity tests: device transfer and the near-tie
rules under which the oracle's integer decisions may differ.

Near-tie rules (from the stated acceptance bar: bit-exact integer outputs
except where the oracle's best two candidates differ by under 1e-6
relative):
  * r*    : the oracle's best two KL values are within 1e-6 relative;
  * tau*  : the oracle's best two E(tau) values are within 1e-6 relative;
  * mask  : the weight lies within 1e-6 sigma of mu +- 3 sigma;
  * codes : the segment's tau* or mask is itself a counted near-tie.
"""
import numpy as np

TIE = 1e-6


def dev(a, torch, bf16: bool):
    """numpy (uint16 bf16 bits or float32) -> torch tensor on cuda:0."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def hessian_err(Hg, Ho):
    """max |dH_ij| / sqrt(H_ii H_jj)."""
    d = np.sqrt(np.maximum(np.diag(Ho), 1e-300))
    return float(np.max(np.abs(Hg.astype(np.float64) - Ho) / (d[:, None] * d[None, :])))


def rel_err(a, b, floor=1e-300):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), floor))) if a.size else 0.0


def kl_near_tie(kl) -> bool:
    s = np.sort(np.asarray(kl))
    return len(s) > 1 and (s[1] - s[0]) <= TIE * max(abs(s[0]), 1e-300)


def compare_sqc(g_out, o_out, group, report=None):
    """Compare SQC outputs; returns the number of excused (near-tie) segments.

    Raises AssertionError on any mismatch that the near-tie rules do not cover."""
    tau_g, tau_o = g_out["tau_idx"], o_out["tau_idx"]
    n, k = tau_o.shape
    margin = o_out["margin"].reshape(n, k, group)
    mask_tie = (margin < TIE).any(axis=-1)
    tau_tie = o_out["gap"] <= TIE
    tie = mask_tie | tau_tie
    bad_tau = (tau_g != tau_o) & ~tie
    assert not bad_tau.any(), f"tau_idx mismatch at {np.argwhere(bad_tau)[:5].tolist()}"
    codes_g = g_out["codes"].reshape(n, k, group)
    codes_o = o_out["codes"].reshape(n, k, group)
    bad_codes = (codes_g != codes_o).any(-1) & ~tie
    assert not bad_codes.any(), f"codes mismatch at segments {np.argwhere(bad_codes)[:5].tolist()}"
    mg = g_out["mask"].view(np.uint32).reshape(n, k, group // 32)
    mo = o_out["mask"].reshape(n, k, group // 32)
    bad_mask = (mg != mo).any(-1) & ~mask_tie
    assert not bad_mask.any(), f"mask mismatch at segments {np.argwhere(bad_mask)[:5].tolist()}"
    same = ~tie
    np.testing.assert_array_equal(g_out["scale"][same], o_out["scale"][same])
    np.testing.assert_array_equal(g_out["zero"][same], o_out["zero"][same])
    excused = int(tie.sum())
    if report is not None:
        report["sqc_near_ties"] = excused
    return excused
