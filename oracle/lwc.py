"""SliM-LLM+: SBA bit-widths with learnable weight clipping in place of SQC.
TEST INFRASTRUCTURE (oracle).

Pages:
* rkmt.cn digest, FAQ on GPTQ / AWQ / OmniQuant: the SliM-LLM+ variant
  replaces SQC with OmniQuant's learnable weight clipping;
* scime.ai summary, opening paragraph and "Key results": an extension with
  gradient-based OmniQuant calibration; SBA added to OmniQuant's learnable
  quantizer;
* briefgpt abstract: SliM-LLM+ extends SliM-LLM with gradient-based
  quantizers.

The pages give no formulas for it.  Learnable weight clipping is restated
here from OmniQuant's published method (Shao et al., ICLR 2024): each
quantization group learns two logits whose sigmoids shrink the group's
maximum and minimum before the min-max quantizer is formed, trained by
gradient descent through a straight-through estimator of the rounding.

Readings taken here (where the pages and that method leave a choice):

* Segments and widths: one clipping pair per row segment (row i, group j,
  the SQC segment), widths from SBA.  b = bits[j], maxq = 2^b - 1.
* Quantizer: SQC's form with the clipped range, float zero point:
      a = sigmoid(gamma), c = sigmoid(beta)
      hi = a * max(w_seg), lo = c * min(w_seg)
      s = (hi - lo) / maxq   (s = 1 when hi - lo <= 0, as min-max does for 0)
      z = -lo / s
      q = clamp(round_half_even(w * (1/s) + z), 0, maxq),  w_hat = (q - z) s
  With a = c = 1 this is the plain min-max quantizer at tau = 1.
* Loss: the layer's output MSE over the calibration tokens,
      L = (1/T) sum_t || x_t W^T - x_t W_hat^T ||^2 = tr(D H D^T) / (2T),
  D = W - W_hat, H = 2 X^T X (the Hessian the path already forms).
* Gradient: straight-through rounding (d round(u)/du = 1) while the rounded
  value lies in [0, maxq]; outside it the clamp passes no gradient.  w is
  not trained (weight clipping only).
* Optimiser: full-batch Adam (beta1 0.9, beta2 0.999, eps 1e-8, no weight
  decay), learning rate 1e-2 and logits initialised to 4.0, OmniQuant's
  settings for the clipping parameters; `iters` steps.  Everything is float64.
* Output: after the last step the clipped range is rounded once to float32
  (lo32 = fl32(c min), hi32 = fl32(a max)) and the float32 min-max quantizer
  of SQC at tau = 1 (its exact operation sequence) gives scale, zero and
  codes, so the result packs and serves like an SQC result.
"""
import numpy as np

from .decode import as_f32, as_f64
from .quantizer import fake_quant, quant_codes

LR = 1e-2
INIT_LOGIT = 4.0
BETA1, BETA2, EPS = 0.9, 0.999, 1e-8


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def clipped_range(wmax, wmin, gamma, beta):
    """(hi, lo, s, z) in float64 for clipping logits gamma, beta [n, k]."""
    hi = sigmoid(gamma) * wmax
    lo = sigmoid(beta) * wmin
    return hi, lo


def quantize_f64(seg, hi, lo, maxq):
    """Float64 forward of the clipped quantizer on segments seg [n, k, g].

    Returns (w_hat, q, inside, s, z); inside marks the weights whose rounded
    value lies in [0, maxq] (the straight-through estimator passes gradient
    there)."""
    spread = hi - lo
    s = np.where(spread > 0, spread / maxq, 1.0)
    z = -lo / s
    u = seg * (1.0 / s)[..., None] + z[..., None]
    qr = np.rint(u)
    inside = (qr >= 0) & (qr <= maxq[..., None])
    q = np.clip(qr, 0, maxq[..., None])
    w_hat = (q - z[..., None]) * s[..., None]
    return w_hat, q, inside, s, z


def loss_from_hessian(W, W_hat, H, T):
    """tr(D H D^T) / (2T) with D = W - W_hat: the mean over the T tokens of
    the squared layer-output error, written with H = 2 X^T X."""
    D = as_f64(W) - np.asarray(W_hat, dtype=np.float64)
    return float(np.einsum("ij,ij->", D @ np.asarray(H, dtype=np.float64), D) / (2.0 * T))


def clip_gradient(W, H, T, bits, gamma, beta, group: int):
    """(loss, dL/dgamma, dL/dbeta) at the given logits (straight-through rounding)."""
    w = as_f64(W)
    n, m = w.shape
    k = m // group
    seg = w.reshape(n, k, group)
    maxq = (2.0 ** np.asarray(bits, dtype=np.float64) - 1.0)[None, :].repeat(n, 0)
    wmax, wmin = seg.max(-1), seg.min(-1)
    a, c = sigmoid(gamma), sigmoid(beta)
    hi, lo = a * wmax, c * wmin
    w_hat, q, inside, s, z = quantize_f64(seg, hi, lo, maxq)
    D = w - w_hat.reshape(n, m)
    P = D @ np.asarray(H, dtype=np.float64)
    loss = float(np.einsum("ij,ij->", D, P) / (2.0 * T))
    G = (-P / T).reshape(n, k, group)            # dL/dw_hat
    # d w_hat / d s and d w_hat / d z per weight
    dws = np.where(inside, -seg / s[..., None] + (q - z[..., None]), q - z[..., None])
    dwz = np.where(inside, 0.0, -s[..., None])
    Gs = (G * dws).sum(-1)
    Gz = (G * dwz).sum(-1)
    live = (hi - lo) > 0                        # s = 1 (fixed) otherwise: no gradient
    # s = (hi - lo)/maxq, z = -lo/s
    ds_dhi, ds_dlo = 1.0 / maxq, -1.0 / maxq
    dz_dhi = lo / (s * s * maxq)
    dz_dlo = -1.0 / s - lo / (s * s * maxq)
    dL_dhi = np.where(live, Gs * ds_dhi + Gz * dz_dhi, 0.0)
    dL_dlo = np.where(live, Gs * ds_dlo + Gz * dz_dlo, 0.0)
    g_gamma = dL_dhi * wmax * a * (1.0 - a)
    g_beta = dL_dlo * wmin * c * (1.0 - c)
    return loss, g_gamma, g_beta


def adam_step(p, g, m1, m2, t, lr=LR):
    """One Adam update (step number t >= 1) of parameters p with gradient g."""
    m1 = BETA1 * m1 + (1.0 - BETA1) * g
    m2 = BETA2 * m2 + (1.0 - BETA2) * (g * g)
    mh = m1 / (1.0 - BETA1 ** t)
    vh = m2 / (1.0 - BETA2 ** t)
    return p - lr * mh / (np.sqrt(vh) + EPS), m1, m2


def final_quantizer(W, bits, gamma, beta, group: int):
    """float32 scale, zero [n, k] and codes [n, m] of the learned clipping:
    the clipped range rounded once to float32, then SQC's float32 min-max
    quantizer at tau = 1."""
    w32 = as_f32(W)
    n, m = w32.shape
    k = m // group
    seg32 = w32.reshape(n, k, group)
    seg = seg32.astype(np.float64)
    a, c = sigmoid(gamma), sigmoid(beta)
    hi32 = (a * seg.max(-1)).astype(np.float32)
    lo32 = (c * seg.min(-1)).astype(np.float32)
    maxq = (np.float32(2.0) ** np.asarray(bits, dtype=np.float32) - np.float32(1.0))[None, :].repeat(n, 0)
    s = (hi32 - lo32) / maxq
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    z = (-lo32 / s).astype(np.float32)
    codes = quant_codes(seg32, s[..., None], z[..., None], maxq[..., None])
    _, w_hat = fake_quant(seg32, s[..., None], z[..., None], maxq[..., None])
    return s, z, codes.reshape(n, m).astype(np.uint8), w_hat.reshape(n, m)


def lwc_calibrate(W, H, T, bits, group: int, iters: int = 20, lr: float = LR, init: float = INIT_LOGIT):
    """Learnable weight clipping for one layer.

    Returns dict: gamma, beta [n, k] float64 after `iters` Adam steps; loss
    [iters + 1] (the float64 loss before each step and after the last);
    scale, zero [n, k] float32; codes [n, m] uint8; w_hat [n, m] float32."""
    n, m = np.shape(W)
    k = m // group
    gamma = np.full((n, k), float(init))
    beta = np.full((n, k), float(init))
    mg, vg = np.zeros((n, k)), np.zeros((n, k))
    mb, vb = np.zeros((n, k)), np.zeros((n, k))
    losses = []
    for t in range(1, iters + 1):
        loss, gg, gb = clip_gradient(W, H, T, bits, gamma, beta, group)
        losses.append(loss)
        gamma, mg, vg = adam_step(gamma, gg, mg, vg, t, lr)
        beta, mb, vb = adam_step(beta, gb, mb, vb, t, lr)
    losses.append(clip_gradient(W, H, T, bits, gamma, beta, group)[0])
    s, z, codes, w_hat = final_quantizer(W, bits, gamma, beta, group)
    return {"gamma": gamma, "beta": beta, "loss": np.array(losses), "scale": s, "zero": z,
            "codes": codes, "w_hat": w_hat}
