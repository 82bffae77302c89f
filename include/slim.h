/*
 * slim.h -- C ABI of the SliM-LLM per-layer quantizer path on gfx950 (MI355X).
 *
 * The path quantizes one linear layer W[n, m] (n outputs, m inputs) from
 * calibration activations X[T, m], as described in "SliM-LLM: Salience-Driven
 * Mixed-Precision Quantization for Large Language Models" (blog digest on
 * rkmt.cn, section "core design": component one SBA and component two SQC;
 * the scime.ai summary, section "Approach"):
 *
 *   slim_hessian        H = 2 X^T X                         (component one, Hessian from calibration)
 *   slim_salience       d = diag((H + a I)^-1), delta = w^2 / d^2, group means   (component one)
 *   slim_salience_u     the same, also writing the upper Cholesky factor of (H + a I)^-1
 *   slim_group_salience the group means from a d already formed (linears sharing H)
 *   slim_sba_search     balanced bit allocation scored by output KL           (component one)
 *   slim_sba_search_ex  the same with an output-MSE objective or a given group order (ablations)
 *   slim_sqc_calibrate  3-sigma mask + tau-grid search of scale and zero       (component two)
 *   slim_gptq_quantize  the same quantizer inside GPTQ's error-compensating sweep  (core design: GPTQ backbone)
 *   slim_gptq_quantize_u  the same with that factor given (no second factorisation)
 *   slim_lwc_calibrate  learnable weight clipping in place of SQC (SliM-LLM+)  (FAQ: GPTQ / AWQ / OmniQuant)
 *   slim_pack           group-structured bit-planes, no bitmap                (FAQ: storage)
 *   slim_qlinear        Y = X W_hat^T read from the planes (decode batches)    (FAQ: deployment)
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers unless the parameter says "host".  Arrays
 *    are dense and row-major; X, W, H, hinv_diag, codes, packed and the
 *    workspace must be 16-byte aligned (SLIM_E_ALIGN otherwise).
 *  - The caller owns all memory.  The library allocates nothing and keeps no
 *    per-call state; scratch memory comes from a caller-provided workspace of
 *    at least the size the matching *_workspace() query returns.  Two
 *    exceptions, both stated where they are declared: the optional kernel
 *    timers (slim_timing_*), which keep process-wide state and create HIP
 *    events while timing is enabled, and slim_qlinear_noalloc, whose scratch
 *    is a fixed device array inside the library.
 *  - Every call enqueues its kernels on `stream` (a hipStream_t passed as
 *    void*, NULL = the default stream) and returns without synchronising.
 *  - Return value: SLIM_OK, or a negative SLIM_E_* code.  Arguments are
 *    checked before anything is enqueued; on an error nothing is enqueued.
 *    After SLIM_E_HIP, slim_last_hip_error() gives the hipError_t (per thread).
 *  - Numeric failures found on the device are reported through a device
 *    int32 `info` word (LAPACK convention): 0 = fine, j > 0 = the leading minor
 *    of order j is not positive definite, -1 = non-finite input.
 *  - Group size g is one of 32, 64, 128 and must divide m.  Average bit-width
 *    N satisfies 2 <= N <= 7 (bit set {N-1, N, N+1}, codes fit in a byte).
 *  - Storage dtypes: SLIM_BF16 (bfloat16 bit patterns) or SLIM_F32.
 *  - Calls on distinct buffers may run concurrently; calls sharing a
 *    workspace must be ordered on one stream.
 */
#ifndef SLIM_H
#define SLIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLIM_VERSION 1

enum slim_status {
  SLIM_OK = 0,
  SLIM_E_NULL = -1,      /* a required pointer is NULL                       */
  SLIM_E_SHAPE = -2,     /* a size is out of range or sizes are inconsistent */
  SLIM_E_DTYPE = -3,     /* unsupported storage dtype                        */
  SLIM_E_PARAM = -4,     /* a hyper-parameter is out of range                */
  SLIM_E_WORKSPACE = -5, /* workspace missing or smaller than required       */
  SLIM_E_HIP = -6,       /* a HIP runtime call or launch failed              */
  SLIM_E_ALIGN = -7      /* a vector-loaded pointer is not 16-byte aligned   */
};

/* Size limits: input width m <= SLIM_MAX_WIDTH; groups per row
 * k = m / g <= SLIM_MAX_GROUPS for the SBA search. */
#define SLIM_MAX_WIDTH 65536
#define SLIM_MAX_GROUPS 2048

typedef enum slim_dtype { SLIM_F32 = 0, SLIM_BF16 = 1 } slim_dtype;

/* Library version (SLIM_VERSION). */
int slim_version(void);

/* Static, human-readable text for a status code (host). */
const char *slim_status_string(int status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int slim_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Hessian proxy (rkmt.cn digest, "core design", component one: the Hessian
 * is estimated from the calibration activations alone, without gradients).
 *
 *   H[m, m] (+)= 2 * X^T X,   X[t, m] token-major in dtype xdt.
 *
 * H is float32, full and exactly symmetric on return.  accumulate = 0
 * overwrites H; accumulate = 1 adds to it (H must then be symmetric on entry,
 * e.g. from a previous call on an earlier token chunk).  t = 0 writes zeros
 * (or leaves H unchanged when accumulating).  The token sum runs in float32
 * on MFMA (bfloat16 or float32 operands as stored) and is reduced over
 * token splits in a fixed order, so results are bitwise reproducible.
 * Requires t >= 0, m >= 1.
 * ---------------------------------------------------------------------- */
size_t slim_hessian_workspace(int64_t t, int64_t m, int xdt);
int slim_hessian(const void *X, int xdt, int64_t t, int64_t m, float *H, int accumulate,
                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Salience (component one: element salience is the SparseGPT elimination
 * error w_ij^2 / [H^-1]_jj^2; scime.ai "Approach": groups are ranked by their
 * average salience).
 *
 *   H_d = H + damp_frac * mean(diag H) * I           (float64)
 *   hinv_diag[j] = [H_d^-1]_jj                       (float64 Cholesky, stored float32)
 *   delta_ij = fl32(fl32(w_ij * w_ij) / fl32(d_j * d_j)),  d = hinv_diag
 *   group_sal[q] = mean of delta over rows 0..n-1, columns q*g .. q*g+g-1
 *                  (float64 sum in a fixed order, stored float64: it decides
 *                  the ranking, so no rounding is added before the search)
 *
 * H: float32 [m, m], symmetric (only the lower triangle is read).
 * W: [n, m] in dtype wdt.  elem_sal: optional float32 [n, m] (NULL = skip).
 * info: device int32, see conventions; outputs are unspecified if info != 0.
 * Requires n >= 1, m >= 1, m % group == 0, damp_frac >= 0.
 * ---------------------------------------------------------------------- */
size_t slim_salience_workspace(int64_t n, int64_t m, int group);
int slim_salience(const float *H, int64_t m, double damp_frac, const void *W, int wdt, int64_t n,
                  int group, float *hinv_diag, double *group_sal, float *elem_sal, int32_t *info,
                  void *ws, size_t ws_bytes, void *stream);

/* slim_salience, and also the upper Cholesky factor U of H_d^-1 (H_d^-1 =
 * U^T U): U float64 [m, m], row-major, zeros below the diagonal, 16-byte
 * aligned.  This is the factor GPTQ's sweep reads (core design: the GPTQ
 * backbone), so slim_gptq_quantize_u can take it instead of factoring H
 * again.  The sweep runs on the index-reversed matrix (its inverse factor,
 * read backwards, is U); hinv_diag, group_sal and elem_sal are the same
 * quantities as slim_salience's, with float64 rounding in another order.
 * U is meaningful only when *info ends 0.  Same workspace as slim_salience.
 */
int slim_salience_u(const float *H, int64_t m, double damp_frac, const void *W, int wdt, int64_t n,
                    int group, float *hinv_diag, double *group_sal, float *elem_sal, double *U,
                    int32_t *info, void *ws, size_t ws_bytes, void *stream);

/* The group-salience half of slim_salience, from a hinv_diag already formed:
 * delta and group_sal exactly as slim_salience forms them from its own
 * hinv_diag, so for the same hinv_diag and W the results are bit-identical.
 * H comes from a layer's input activations (component one), so the linears
 * that read the same input share H and d: one slim_salience per input width
 * gives hinv_diag, and the other linears of that width call this instead of
 * factoring H again.
 * hinv_diag: float32 [m] (slim_salience's, or any positive d).  W: [n, m] in
 * dtype wdt.  group_sal: float64 [m/group].  elem_sal: optional float32
 * [n, m] (NULL = skip).  info: device int32, written 0, or -1 if W holds a
 * non-finite value (then group_sal is unspecified).
 * Requires n >= 1, m >= 1, m % group == 0.
 */
size_t slim_group_salience_workspace(int64_t n, int64_t m, int group);
int slim_group_salience(const float *hinv_diag, int64_t m, const void *W, int wdt, int64_t n, int group,
                        double *group_sal, float *elem_sal, int32_t *info, void *ws, size_t ws_bytes,
                        void *stream);

/* ------------------------------------------------------------------------
 * SBA search (component one: bit-widths minimise the KL divergence of the
 * layer output under |G_{N-1}| = |G_{N+1}|, searched by two pointers over
 * [0, k/2]).
 *
 * Groups are ranked by descending group_sal (ties: lower index first).  For
 * every step r = 0 .. floor(k/2) the first r ranked groups get N+1 bits, the
 * last r get N-1 and the rest N.  Each step's trial weights are the min-max
 * quantizer at tau = 1 per row segment, stored back in dtype wdt, and the
 * step is scored by
 *     kl[r] = mean_t KL( softmax_j(x_t W^T) || softmax_j(x_t W_r^T) )
 * (softmax over the n outputs, natural log).  r_star = first argmin of kl;
 * bits[q] is the allocation at r_star.
 *
 * X: [t, m] (dtype xdt), W: [n, m] (dtype wdt == xdt); group_sal float64 [k];
 * bits int8 [k]; kl float64 [floor(k/2)+1]; r_star int32 [1].
 * Requires t >= 1, n >= 1, m % group == 0, k <= SLIM_MAX_GROUPS and
 * 3 * n * m * sizeof(element) < 2^31 (the trial weights are addressed with
 * 32-bit offsets; 28672 x 8192 bf16 uses 1.4 GB).
 *
 * Workspace: slim_sba_workspace() gives the size that lets the tokens run in
 * batches of up to 4 GB of per-token softmax statistics.  A smaller ws_bytes
 * is accepted down to the size that holds one 256-token tile per batch: the
 * tokens are then split into more batches (same result up to float rounding
 * order inside each token's statistics, which do not depend on the batch);
 * below that the call returns SLIM_E_WORKSPACE.
 *
 * With bf16 operands, the KL objective, g = 64 or 128 and an even number of
 * 64-column stages over m, the scan reduces half of a step's softmax
 * statistics (one token block of each tile) during the next step's matrix
 * products, the other half right after the step's own; the results are
 * bit-identical to the plain scan, which the environment variable
 * SLIM_SBA_NO_OVERLAP (any
 * value, read at each call) selects instead.
 * ---------------------------------------------------------------------- */
size_t slim_sba_workspace(int64_t t, int64_t n, int64_t m, int group, int dtype);
int slim_sba_search(const void *X, int xdt, int64_t t, const void *W, int wdt, int64_t n, int64_t m,
                    int group, const double *group_sal, int avg_bits, int8_t *bits, double *kl,
                    int32_t *r_star, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * SBA search variants for the ablations (scime.ai summary, "Measured
 * effects": KL rather than MSE as the objective; random or head-tail group
 * allocation instead of the salience ranking; rkmt.cn digest, Fig. 5).
 *
 * As slim_sba_search, with two changes:
 *  - order (device int32 [k], or null): when given, it replaces the salience
 *    ranking: step r raises order[0 .. r-1] and lowers order[k-r .. k-1]
 *    (group_sal is then ignored and may be null).  It must be a permutation
 *    of 0 .. k-1; entries outside that range are read as group 0 (the scan
 *    stays in bounds, its result is meaningless).  Head-tail is the identity
 *    order, random a permutation the caller draws.
 *  - objective: SLIM_OBJ_KL (0) scores steps as slim_sba_search does;
 *    SLIM_OBJ_MSE (1) scores them by the squared output error
 *        score[r] = mean_t || x_t W^T - x_t W_r^T ||^2   (sum over the n outputs).
 * score float64 [floor(k/2)+1]; r_star is its first argmin.  Errors as for
 * slim_sba_search, plus SLIM_E_PARAM for an unknown objective and SLIM_E_NULL
 * when both group_sal and order are null.
 * ---------------------------------------------------------------------- */
#define SLIM_OBJ_KL 0
#define SLIM_OBJ_MSE 1
int slim_sba_search_ex(const void *X, int xdt, int64_t t, const void *W, int wdt, int64_t n, int64_t m,
                       int group, const double *group_sal, const int32_t *order, int avg_bits, int objective,
                       int8_t *bits, double *score, int32_t *r_star, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * SQC calibration (component two: salient weights outside mu +- 3 sigma and
 * the rest share one quantizer; tau scales its scale and zero over n_tau + 1
 * linear candidates in [1 - lambda, 1 + lambda]; the candidate with the
 * smallest salience-weighted l2 error wins; no parameter is added).
 *
 * Per row segment (row i, group q, b = bits[q], maxq = 2^b - 1):
 *   lo/hi = min/max; s0 = (hi-lo)/maxq (1 if 0); z0 = -lo/s0       (float32)
 *   mask  = w < mu - 3 sigma  or  w > mu + 3 sigma  (population sigma, float64)
 *   for tau_i = 1 + lambda (2i - n_tau)/n_tau:  s = tau s0, z = tau z0,
 *       q = clamp(rint(w * (1/s) + z), 0, maxq), e = w - (q - z) s   (float32, no FMA)
 *       E_i = mean_{mask}(delta e^2) + mean_{~mask}(delta e^2)     (float64)
 *   tau* = first argmin E;  scale = tau* s0, zero = tau* z0, codes at tau*.
 *
 * W: [n, m] (dtype wdt); bits int8 [k]; hinv_diag float32 [m] (delta as in
 * slim_salience); scale, zero float32 [n, k]; codes uint8 [n, m];
 * mask uint32 [n, m/32] (bit c of word w of row i <-> column 32w + c);
 * tau_idx uint8 [n, k] or NULL.  Requires 1 <= n_tau <= 255, lambda in
 * [0, 1), bits[q] in [1, 8].  n = 0 is a no-op.
 * ---------------------------------------------------------------------- */
int slim_sqc_calibrate(const void *W, int wdt, int64_t n, int64_t m, int group, const int8_t *bits,
                       const float *hinv_diag, double lambda, int n_tau, float *scale, float *zero,
                       uint8_t *codes, uint32_t *mask, uint8_t *tau_idx, void *stream);

/* The tau candidates slim_sqc_calibrate uses, written to host memory
 * out_host[0 .. n_tau] (float64 evaluation rounded once to float32). */
int slim_tau_table(double lambda, int n_tau, float *out_host);

/* ------------------------------------------------------------------------
 * GPTQ sweep with the SliM-LLM group quantizer (rkmt.cn digest, core design
 * and the FAQ on GPTQ / AWQ / OmniQuant: SliM-LLM plugs SBA and SQC into
 * GPTQ's layer-wise backbone; GPTQ, Frantar et al., ICLR 2023).
 *
 * Columns are quantized in order.  With H_d = H + damp_frac * mean(diag H) * I
 * and U the upper Cholesky factor of H_d^-1 (H_d^-1 = U^T U), after column c
 *     e_c = (w_c - w_hat_c) / U_cc,   w_c' -= e_c U[c, c']  for every c' > c,
 * in float64.  Group q's quantizer is fixed when the sweep reaches its first
 * column: the slim_sqc_calibrate calibration (same lambda, n_tau, hinv_diag)
 * of the group's current weights rounded to float32, at width bits[q].
 * Each column's code is that quantizer's float32 decision on its current
 * weight rounded to float32; w_hat = (q - zero) * scale.
 *
 * H: float32 [m, m] (slim_hessian's output, undamped); W: [n, m] (dtype
 * wdt); bits int8 [k] (widths in [1, 8], e.g. from slim_sba_search);
 * hinv_diag float32 [m] (slim_salience's, same damp_frac).  Outputs: scale,
 * zero float32 [n, k]; codes uint8 [n, m]; mask uint32 [n, m/32] (the
 * 3-sigma mask of each group's calibration); tau_idx uint8 [n, k] or NULL;
 * info int32 [1] (LAPACK convention for H_d; -1 for non-finite H or W;
 * outputs unspecified when info != 0).  Workspace:
 * slim_gptq_workspace(n, m, g) bytes (8 (2 m_p^2 + n m) + 4 n m bytes
 * and change, m_p = m rounded up to 64).  Requires n >= 1, m % group == 0,
 * damp_frac >= 0, the lambda / n_tau ranges of slim_sqc_calibrate.
 * ---------------------------------------------------------------------- */
size_t slim_gptq_workspace(int64_t n, int64_t m, int group);
int slim_gptq_quantize(const float *H, int64_t m, double damp_frac, const void *W, int wdt, int64_t n, int group,
                       const int8_t *bits, const float *hinv_diag, double lambda, int n_tau, float *scale,
                       float *zero, uint8_t *codes, uint32_t *mask, uint8_t *tau_idx, int32_t *info, void *ws,
                       size_t ws_bytes, void *stream);

/* slim_gptq_quantize with the factor given: U float64 [m, m] as
 * slim_salience_u writes it (16-byte aligned; read only).  H and damp_frac
 * are not needed; *info is set to 0, or -1 for a non-finite W.  Same
 * workspace and outputs as slim_gptq_quantize, which, given the same H, forms
 * the same U itself. */
int slim_gptq_quantize_u(const double *U, int64_t m, const void *W, int wdt, int64_t n, int group,
                         const int8_t *bits, const float *hinv_diag, double lambda, int n_tau, float *scale,
                         float *zero, uint8_t *codes, uint32_t *mask, uint8_t *tau_idx, int32_t *info, void *ws,
                         size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * SliM-LLM+: learnable weight clipping in place of SQC (rkmt.cn digest, FAQ
 * on GPTQ / AWQ / OmniQuant: SliM-LLM+ replaces SQC with OmniQuant's
 * learnable weight clipping; scime.ai summary, opening paragraph and "Key
 * results": gradient-based calibration with SBA's widths).
 *
 * Per row segment (row i, group q, b = bits[q], maxq = 2^b - 1), two logits
 * gamma, beta (start value `init`) clip the segment's range, float64:
 *   hi = sigmoid(gamma) max(w), lo = sigmoid(beta) min(w),
 *   s = (hi - lo)/maxq (1 if hi <= lo), z = -lo/s,
 *   w_hat = (clamp(rint(w (1/s) + z), 0, maxq) - z) s.
 * They are trained for `iters` full-batch Adam steps (beta1 0.9, beta2
 * 0.999, eps 1e-8, learning rate lr) on the layer's output MSE over the
 * t_tokens calibration tokens, L = tr((W - W_hat) H (W - W_hat)^T) / (2 t),
 * through a straight-through rounding (no gradient where the clamp holds).
 * H is the slim_hessian output for those tokens (float32 [m, m], symmetric;
 * only the lower triangle is read).  Then the
 * clipped range is rounded once to float32 and SQC's float32 min-max
 * quantizer at tau = 1 gives scale, zero (float32 [n, k]) and codes (uint8
 * [n, m]), which slim_pack and slim_qlinear take as they take SQC's.
 * loss: float64 [iters + 1], L before each step and after the last;
 * logits: float64 [2, n, k] (gamma, then beta) or NULL.  W: [n, m] in dtype
 * wdt.  Requires 0 <= iters <= SLIM_LWC_MAX_ITERS, lr > 0.  Workspace:
 * slim_lwc_workspace(n, m, g, iters) bytes (float64 copies of W - W_hat and
 * of H, padded to multiples of 64, the float64 product [n, m], and
 * per-segment state).
 * ---------------------------------------------------------------------- */
#define SLIM_LWC_MAX_ITERS 10000
size_t slim_lwc_workspace(int64_t n, int64_t m, int group, int iters);
int slim_lwc_calibrate(const void *W, int wdt, int64_t n, int64_t m, int group, const int8_t *bits, const float *H,
                       int64_t t_tokens, int iters, double lr, double init, float *scale, float *zero,
                       uint8_t *codes, double *logits, double *loss, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Packing (FAQ on storage: group-wise bit-widths need no bitmap or codebook
 * and no extra storage; dequantization keeps the uniform-quantizer form).
 *
 * Bit-planes, group-major.  Group q starts at word off(q) = n (g/32) *
 * sum_{q' < q} bits[q'];  word (q, plane p, row i, w) is at off(q) +
 * (p n + i)(g/32) + w; its bit c is bit p of codes[i, q g + 32 w + c].
 * packed: uint32 [n m avg_bits / 32] (slim_pack_words).  Bits above bits[q]
 * in a code are ignored.  If bits[q] leaves [1, 8] or the widths do not sum to
 * k * avg_bits, *info (device int32, may be NULL) is set to 1 and no word
 * outside `packed` is written.  n = 0 is a no-op.
 * ---------------------------------------------------------------------- */
int64_t slim_pack_words(int64_t n, int64_t m, int avg_bits);
int slim_pack(const uint8_t *codes, int64_t n, int64_t m, int group, const int8_t *bits,
              int avg_bits, uint32_t *packed, int32_t *info, void *stream);

/* ------------------------------------------------------------------------
 * Mixed-precision linear layer on the packed planes (rkmt.cn digest, FAQ on
 * storage and deployment: no bitmap or codebook, dequantization with the
 * structure of uniform quantization; scime.ai summary, "Limitations": the
 * speed of mixed-precision dequantization at inference).
 *
 *   Y[a, i] = sum_c X[a, c] * (q[i, c] - zero[i, c/g]) * scale[i, c/g]
 *
 * q is decoded from packed (the slim_pack layout, widths bits[k]); scale and
 * zero are the float32 [n, k] outputs of slim_sqc_calibrate.  X: [t, m] in
 * dtype xdt (bfloat16 or float32), 1 <= t <= SLIM_QLINEAR_MAX_T (decode
 * batches and prefill); Y: float32 [t, n].  Accumulation is float32; for a
 * given t the sum over groups runs in a fixed order (bitwise reproducible).
 * Up to two tokens the codes are summed through nibble tables; from three
 * to eight they are expanded to bfloat16 integers for the matrix cores
 * (float32 X as three exact bfloat16 terms); above eight a GEMM over the
 * planes expands each code once per 128 tokens.  Results for different t
 * agree to float32 rounding, not bit for bit.  bits must
 * hold widths in 1 .. 8 adding up to k * avg_bits, as slim_pack requires;
 * otherwise every output is NaN (checked before any plane is read).  Workspace:
 * slim_qlinear_workspace(t, n, m, g) bytes (partial sums over runs of
 * groups when the layer is split along its input, or the group sums of X for
 * t > 8; its contents on entry do not matter).
 * ---------------------------------------------------------------------- */
#define SLIM_QLINEAR_MAX_T 65536
size_t slim_qlinear_workspace(int64_t t, int64_t n, int64_t m, int group);
int slim_qlinear(const void *X, int xdt, int64_t t, int64_t m, const uint32_t *packed, const int8_t *bits,
                 int avg_bits, const float *scale, const float *zero, int64_t n, int group, float *Y, void *ws,
                 size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * slim_qlinear without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * Same arguments, computation and results as slim_qlinear (bit for bit: the
 * same plan and kernels) without ws / ws_bytes.  The partial sums go to a
 * device array of SLIM_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library's
 * code object, which every GPU the library runs on holds from module load
 * until the process ends; the call itself allocates nothing and records no
 * timing events.  Its device address is looked up on the first call on each
 * device (with that device current).  A layer whose partial sums need more
 * than the array (slim_qlinear_workspace(t, n, m, g) >
 * SLIM_NOALLOC_SCRATCH_BYTES) gets SLIM_E_WORKSPACE before anything is
 * enqueued.  Nothing in the array has to start at zero: every call writes the
 * partial sums it reads.  The array is shared by all calls on one GPU and
 * keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or from host threads without ordering) race on it and
 * their results are undefined, so order them on one stream.  The call runs on
 * the current device; `stream` must belong to it.
 * ---------------------------------------------------------------------- */
#define SLIM_NOALLOC_SCRATCH_BYTES (32u << 20)
size_t slim_qlinear_noalloc_scratch_bytes(void);
int slim_qlinear_noalloc(const void *X, int xdt, int64_t t, int64_t m, const uint32_t *packed, const int8_t *bits,
                         int avg_bits, const float *scale, const float *zero, int64_t n, int group, float *Y,
                         void *stream);

/* ------------------------------------------------------------------------
 * Kernel timing (instrumentation, not part of the method).  When enabled,
 * the library records a pair of HIP events on the launch stream around every
 * launch of the named kernels: "hessian_gram", "chol_update", "sba_klgemm",
 * "sqc_calibrate", "pack_planes", "qlinear" (its one or two kernels),
 * "gptq_sweep", "gptq_trail" (per group), "lwc_dh" (the product D H of each
 * learnable-clipping iteration).
 * slim_timing_read synchronises those events
 * and returns the summed milliseconds and the launch count since the last
 * reset.  Returns SLIM_E_PARAM for an unknown name.  slim_timing_enable(1)
 * selects every kernel; slim_timing_select then leaves one out (on = 0) or
 * takes it back, so that kernels launched many times per call (chol_update,
 * gptq_sweep, gptq_trail: per panel or per group) need not add their event
 * records to a timed run.  The timers are process-wide state: while timing is
 * enabled every timed launch creates two HIP events (destroyed when read).
 * ---------------------------------------------------------------------- */
int slim_timing_enable(int on);
int slim_timing_select(const char *kernel, int on);
int slim_timing_reset(void);
int slim_timing_read(const char *kernel, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* SLIM_H */
