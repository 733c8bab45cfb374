/*
 * kla.h — C ABI of the Kalman Linear Attention (KLA) forward scan for AMD
 * MI355X (gfx950).
 *
 * Method (gist.science summaries of arXiv 2602.10743, "Kalman Linear
 * Attention"; [KLA-nl] = "Technische Samenvatting: Kalman Linear Attention
 * (KLA)"): sequence mixing as exact Bayesian filtering in a diagonal
 * linear-Gaussian state-space model.  Per head (b,h), key channel i and value
 * channel j, one scalar filter:
 *
 *   prior   x_t = a_t x_{t-1} + w_t, w_t ~ N(0, pbar_t), a_t = exp(log_decay_t)
 *           ([KLA-nl] §1, "Dynamics Prior": exactly discretised OU process)
 *   evidence v_{t,j} = k_{t,i} x_{t,ij} + e, e of precision Lambda^v_{t,i}
 *           ([KLA-nl] §1, "Observatiemodel")
 *   output  y_{t,j} = sum_i q_{t,i} mu_{t,ij} (posterior mean; §1 "Readout")
 *
 * The posterior precision follows the Möbius map of [KLA-nl] §2
 * ("Parallelisatie via Möbius-transformaties", precision equation)
 *   lambda_t = ((1 + c pbar) lambda_{t-1} + c a^2) / (pbar lambda_{t-1} + a^2),
 *   c = k^2 Lambda^v,
 * evaluated as a scan of 2x2 projective matrices; the posterior mean follows
 * the affine recursion mu_t = f_t mu_{t-1} + g_t v_t with the precision-ratio
 * gates f = a lambda^-_t / lambda_t and g = k Lambda^v / lambda_t ([KLA-nl] §3,
 * "Niet-lineaire Gating vanuit Onzekerheid").
 *
 * Conventions for every entry point:
 *   - All tensors are dense, row-major, on the device, not aliased (unless an
 *     entry point allows it), and owned by the caller.  The library never
 *     allocates or frees device memory (the scratch array of
 *     kla_forward_noalloc is part of its code object, placed by the HIP
 *     loader) and never synchronises (kla_workspace_error excepted); work is
 *     enqueued on `stream` (a hipStream_t; NULL
 *     means the default stream) and the call returns without waiting.
 *   - Argument validation happens on the host before any HIP call; a
 *     non-zero return means nothing was enqueued.  KLA_ERR_HIP means a launch
 *     failed; kla_status_string() then returns the HIP error text.
 *   - Device data is not checked: lambda0 must be positive and every input
 *     finite, otherwise outputs are unspecified (typically NaN).  The
 *     precision is carried in float32 and must stay below FLT_MAX: with
 *     proc_noise > 0 it is bounded by c + 1/proc_noise, but with proc_noise = 0
 *     and a < 1 it grows by 1/a^2 per token and overflows after about
 *     88 / ln(1/a^2) tokens, after which outputs are unspecified.
 *   - A workspace is device memory of at least the size the matching
 *     *_workspace_bytes() function returns, 256-byte aligned, zero-filled once
 *     by kla_workspace_init() before its first use and not touched by the
 *     caller afterwards.  Calls that share one workspace must be ordered on one
 *     stream; concurrent calls on one workspace race.  A workspace serves one
 *     entry point only (kla_forward, kla_forward_ou and kla_forward_prologue
 *     count as one): the entry points keep different flags and counters in
 *     it, so a buffer used by kla_forward must not be passed to
 *     kla_precision_scan or kla_backward, and so on.
 */
#ifndef KLA_H_
#define KLA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KLA_F32 = 0, KLA_BF16 = 1 } kla_dtype;

typedef enum {
  KLA_OK = 0,
  KLA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, bad alignment        */
  KLA_ERR_UNSUPPORTED = 2,  /* d_k / d_v / dtype outside the supported set  */
  KLA_ERR_WORKSPACE = 3,    /* workspace missing, misaligned or too small   */
  KLA_ERR_HIP = 4,          /* a HIP call failed (text via status string)   */
  KLA_ERR_TOO_LARGE = 5     /* kla_forward_noalloc: the shape needs more
                               than KLA_NOALLOC_SCRATCH_BYTES of scratch    */
} kla_status;

/* Bytes of workspace kla_forward needs for this shape; 0 if the shape is
 * invalid or unsupported. */
size_t kla_forward_workspace_bytes(int B, int H, int T, int dk, int dv);

/*
 * KLA forward pass over T tokens of B*H independent heads.
 *
 * Inputs (dtype = KLA_BF16: bfloat16 values; KLA_F32: float32):
 *   q, k, log_decay, proc_noise, val_prec   [B,H,T,dk]
 *   v                                       [B,H,T,dv]
 *   log_decay is log a_t (a_t = exp(log_decay) <= 1 expected), proc_noise is
 *   the process-noise variance pbar_t >= 0, val_prec is Lambda^v_t >= 0.
 * State in (float32, nullable):
 *   lambda0 [B,H,dk]      posterior precision before token 1 (NULL: all 1)
 *   M0      [B,H,dk,dv]   posterior mean before token 1     (NULL: all 0)
 * Outputs:
 *   y          [B,H,T,dv]  dtype; readout of the posterior mean after token t
 *   lambda_T   [B,H,dk]    float32 precision after the last token
 *   M_T        [B,H,dk,dv] float32 posterior mean after the last token
 *   lambda_path [B,H,T,dk] float32 precision after every token (NULL: skipped)
 * (lambda_T, M_T) fed back as (lambda0, M0) continue the scan exactly: two
 * calls over T1 and T2 tokens equal one call over T1 + T2 up to rounding.
 * T = 0 copies the state in to the state out; the per-token arrays are then
 * not accessed and may be NULL.
 *
 * Supported: dk, dv in {16, 32, 64, 128}; B, H >= 1; T >= 0;
 * B*H*T*max(dk,dv) < 2^31.  Arithmetic: float32 gates and scan; the bf16 path
 * feeds the chunk contractions to bf16 matrix cores with float32 accumulation.
 */
int kla_forward(const void* q, const void* k, const void* v,
                const void* log_decay, const void* proc_noise, const void* val_prec,
                const float* lambda0, const float* M0,
                void* y, float* lambda_T, float* M_T, float* lambda_path,
                int B, int H, int T, int dk, int dv, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device scratch array inside the library that
 * kla_forward_noalloc works in (one array per GPU). */
#define KLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * kla_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Inputs, outputs, shapes, dtypes, alignment rules and results are those of
 * kla_forward (same kernels); the workspace is replaced by a file-scope device
 * array of KLA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU,
 * which that GPU holds until the process ends.  The call allocates nothing
 * (no hipMalloc / hipFree, no allocating library routine).
 *
 * Per call, on `stream`: a fill kernel clears the scratch's control words and
 * carry flags (every call starts as on a freshly initialised workspace), then
 * kla_forward's kernels run.  The first call on a device looks up the array's
 * device address there (that device current) and keeps it for later calls.
 *
 * error_flag: nullable device pointer to one int (4-byte aligned).  When
 *   given, a one-thread kernel on `stream` writes this call's device error
 *   word there after the call's kernels: 0 = none, 1 = as kla_workspace_error
 *   reports it (a look-back gave up waiting; outputs unspecified).
 * Errors: KLA_ERR_TOO_LARGE when this shape needs more scratch than
 *   KLA_NOALLOC_SCRATCH_BYTES (nothing is launched; kla_forward with a
 *   workspace serves every shape); otherwise as kla_forward.  The run kernel
 *   (bf16, dk = dv = 64) fits up to about 1900 (head, run) pairs, e.g.
 *   B*H = 64 at T = 2048 or B*H = 192 at T = 2048; the segment kernels fit
 *   B*H*ceil(T/64) up to about 2000 at dk = dv = 64.
 * Concurrency: every call on one GPU shares that GPU's array and leaves its
 *   contents behind: calls that overlap on one GPU (two streams, two threads,
 *   two graph replays in flight) race and give unspecified results.  Order
 *   them on one stream.
 */
int kla_forward_noalloc(const void* q, const void* k, const void* v,
                        const void* log_decay, const void* proc_noise, const void* val_prec,
                        const float* lambda0, const float* M0,
                        void* y, float* lambda_T, float* M_T, float* lambda_path,
                        int B, int H, int T, int dk, int dv, int dtype,
                        int* error_flag, void* stream);

/*
 * KLA forward pass with the OU prior given in continuous time: the same scan
 * as kla_forward, with log_decay and proc_noise formed inside the kernel by the
 * exact discretisation of an Ornstein-Uhlenbeck step ([KLA-nl] §1, "Dynamics
 * Prior": the prior is an exactly discretised OU process):
 *   a_t   = exp(-theta dt_t)                        (log_decay = -theta dt_t)
 *   pbar_t = sigma2 (1 - exp(-2 theta dt_t)) / (2 theta)   (-> sigma2 dt_t as theta -> 0)
 * per (b,h,t,i), with theta and sigma2 per (h,i).  One per-token coefficient
 * stream (dt) replaces two (log_decay, proc_noise).
 *
 * Inputs: q, k, val_prec [B,H,T,dk] and v [B,H,T,dv] as kla_forward;
 *   dt     [B,H,T,dk] dtype, the step length of each token and channel (>= 0);
 *   theta  [H,dk]     float32, OU rate (mean reversion), shared over the batch;
 *   sigma2 [H,dk]     float32, OU diffusion (variance per unit time, >= 0).
 * State, outputs, workspace (kla_forward_workspace_bytes; the layout is
 * kla_forward's, so one workspace may serve both), supported shapes and
 * errors: as kla_forward.  theta and sigma2 need 4-byte alignment.
 */
int kla_forward_ou(const void* q, const void* k, const void* v, const void* dt,
                   const float* theta, const float* sigma2, const void* val_prec,
                   const float* lambda0, const float* M0,
                   void* y, float* lambda_T, float* M_T, float* lambda_path,
                   int B, int H, int T, int dk, int dv, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * KLA forward pass behind its coefficient prologue: the scan of
 * kla_forward_ou fed from raw projections, as in a Mamba-like block
 * ([KLA-nl] §4 "Architectuur": the scan sits between causal 1D convolutions
 * with SiLU activations; §1 "Dynamics Prior": exactly discretised OU prior).
 * Per (b,h,t) and channel c, inside the kernel:
 *   u_t[c]  = b[h,c] + sum_{s<W} w[h,c,s] x_{t-(W-1)+s}[c]   (x_t = 0 for t < 0)
 *   q, k, v = SiLU(u) = u / (1 + e^{-u}) of xq, xk, xv, each with its own
 *             taps, held in the input dtype (bf16: rounded to nearest even)
 *   dt       = softplus(dt_raw),  Lambda^v = softplus(vp_raw)   (float32)
 *   log_decay, proc_noise from (theta, sigma2, dt) as kla_forward_ou.
 * The convolution starts from zero history at t = 0: a call covers a whole
 * sequence (no convolution state is carried between calls; lambda0 / M0 still
 * continue the filter).
 *
 * Inputs: xq, xk, dt_raw, vp_raw [B,H,T,dk] and xv [B,H,T,dv] (dtype, 16-byte
 *   aligned); theta, sigma2 [H,dk] float32 as kla_forward_ou;
 *   conv_wq, conv_wk [H,dk,W] and conv_wv [H,dv,W] float32 taps (tap W-1
 *   multiplies the current token; 16-byte aligned; the layout of a depthwise
 *   torch Conv1d weight [channels,1,W] per head);
 *   conv_bq, conv_bk [H,dk], conv_bv [H,dv] float32 biases, nullable (zero);
 *   conv_width W in 1..4.
 * State, outputs, workspace (kla_forward_workspace_bytes; the layout is
 * kla_forward's), supported shapes and errors: as kla_forward.
 */
int kla_forward_prologue(const void* xq, const void* xk, const void* xv, const void* dt_raw,
                         const float* theta, const float* sigma2, const void* vp_raw,
                         const float* conv_wq, const float* conv_wk, const float* conv_wv,
                         const float* conv_bq, const float* conv_bk, const float* conv_bv, int conv_width,
                         const float* lambda0, const float* M0,
                         void* y, float* lambda_T, float* M_T, float* lambda_path,
                         int B, int H, int T, int dk, int dv, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * KLA with the value precision indexed by value channel: val_prec is
 * [B,H,T,dv] (Lambda^v_{t,j}) instead of [B,H,T,dk], so every element (i, j)
 * is its own scalar filter with observation precision c = k_{t,i}^2
 * Lambda^v_{t,j} ([KLA-nl] §1 "Observatiemodel" read with Lambda^v per value
 * channel; predict/update of §2 and precision-ratio gates of §3 per element):
 *   precision lam_{t,ij}, gates f_{t,ij}, g_{t,ij}, mean M_{t,ij},
 *   y_t[j] = sum_i q_{t,i} M_{t,ij}.
 * Inputs: q, k, log_decay, proc_noise [B,H,T,dk]; v, val_prec [B,H,T,dv]
 * (dtype); state in lambda0, M0 [B,H,dk,dv] float32, nullable (1 and 0).
 * Outputs: y [B,H,T,dv] dtype; lambda_T, M_T [B,H,dk,dv] float32.  T = 0
 * copies the state in to the state out.  No workspace: one kernel walks the
 * sequence per element.  Supported: dk, dv in {16, 32, 64, 128};
 * B*H*T*max(dk,dv) < 2^31.  Alignment: element size (float32 arrays 4 bytes).
 * Arithmetic: float32; the readout sums over key channels in a fixed order.
 */
int kla_forward_vprec(const void* q, const void* k, const void* v,
                      const void* log_decay, const void* proc_noise, const void* val_prec,
                      const float* lambda0, const float* M0,
                      void* y, float* lambda_T, float* M_T,
                      int B, int H, int T, int dk, int dv, int dtype, void* stream);

/* Bytes of workspace kla_precision_scan needs; 0 if the shape is invalid. */
size_t kla_precision_scan_workspace_bytes(int B, int H, int T, int D);

/*
 * Precision path only: B*H*D independent Möbius chains of length T
 * ([KLA-nl] §2, precision equation), float32 throughout.
 *   log_decay, proc_noise, obs_prec [B,H,T,D]   obs_prec = c_t = k_t^2 Lambda^v_t
 *   lambda0     [B,H,D]   nullable (NULL: all 1)
 *   lambda_path [B,H,T,D] precision after every token (required)
 *   lambda_T    [B,H,D]   precision after the last token (nullable)
 * Supported: D >= 1, B*H*T*D < 2^62, B*H*D < 2^31.  With T = 0 only lambda0
 * and lambda_T are accessed (the other arrays may be NULL).
 */
int kla_precision_scan(const float* log_decay, const float* proc_noise, const float* obs_prec,
                       const float* lambda0, float* lambda_path, float* lambda_T,
                       int B, int H, int T, int D,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode: one filter step per head, for generating token by token.  The same
 * step the forward pass takes for every token ([KLA-nl] §2: precision
 * equation and affine mean recursion; §3: precision-ratio gates; §1: readout
 * of the posterior mean), applied to the state the caller carries.
 *
 * Inputs (dtype = KLA_BF16: bfloat16 values; KLA_F32: float32), one token:
 *   q, k, log_decay, proc_noise, val_prec   [B,H,dk]
 *   v                                       [B,H,dv]
 * State before the token (float32, nullable):
 *   lambda_in [B,H,dk]     posterior precision (NULL: all 1, the prior)
 *   M_in      [B,H,dk,dv]  posterior mean      (NULL: all 0, the prior)
 * Outputs:
 *   lambda_out [B,H,dk]     float32 precision after the token
 *   M_out      [B,H,dk,dv]  float32 posterior mean after the token
 *   y          [B,H,dv]     dtype; readout q^T M_out
 * The state may be updated in place: lambda_out may equal lambda_in and M_out
 * may equal M_in (the same pointer); any other overlap between arguments is
 * not allowed.  Starting from (lambda0, M0), T calls reproduce kla_forward
 * over the same T tokens up to rounding.  No workspace: one kernel, no state
 * kept between calls.
 *
 * Supported: dk, dv in {16, 32, 64, 128}; 1 <= B*H < 2^31.  Alignment:
 * M_in and M_out 16 bytes, the other arrays their element size.
 * Arithmetic: float32 throughout.
 */
int kla_decode_step(const void* q, const void* k, const void* v,
                    const void* log_decay, const void* proc_noise, const void* val_prec,
                    const float* lambda_in, const float* M_in,
                    float* lambda_out, float* M_out, void* y,
                    int B, int H, int dk, int dv, int dtype, void* stream);

/* Bytes of workspace kla_backward needs for this shape; 0 if the shape is
 * invalid or unsupported. */
size_t kla_backward_workspace_bytes(int B, int H, int T, int dk, int dv);

/*
 * KLA backward pass: the gradients of a scalar loss L with respect to every
 * input of kla_forward, given dL/dy, dL/dlambda_T and dL/dM_T.  Training KLA
 * as a sequence mixer needs them ([KLA-nl] "Belangrijkste Bijdragen"); the
 * step that is differentiated is the filter step of [KLA-nl] §2 (precision
 * equation, affine mean recursion) with the precision-ratio gates of §3.
 *
 * Inputs: the forward call's q, k, v, log_decay, proc_noise, val_prec (dtype,
 * shapes as kla_forward), lambda0 [B,H,dk] and M0 [B,H,dk,dv] (float32,
 * nullable: 1 and 0 as in kla_forward), and
 *   lambda_path   [B,H,T,dk] float32, the precision path kla_forward wrote
 *                 (its lambda_path output) for these inputs and lambda0;
 *   grad_y        [B,H,T,dv] dtype, dL/dy;
 *   grad_lambda_T [B,H,dk]    float32, dL/dlambda_T (nullable: 0);
 *   grad_M_T      [B,H,dk,dv] float32, dL/dM_T      (nullable: 0).
 * Outputs (overwritten):
 *   grad_q, grad_k, grad_log_decay, grad_proc_noise, grad_val_prec
 *                 [B,H,T,dk] dtype;
 *   grad_v        [B,H,T,dv] dtype;
 *   grad_lambda0  [B,H,dk]    float32;
 *   grad_M0       [B,H,dk,dv] float32.
 * The mean M is recomputed from (lambda_path, inputs, M0); nothing else is
 * saved from the forward call.  T = 0 gives grad_lambda0 = grad_lambda_T and
 * grad_M0 = grad_M_T (zero where those are NULL); the per-token arrays are
 * then not accessed and may be NULL.
 *
 * Supported: dk, dv in {16, 32, 64, 128} (a width of 128 runs as two 64-wide
 * halves); B, H >= 1; T >= 0; B*H*T*max(dk,dv) < 2^31.  Alignment: the per-token arrays (inputs,
 * lambda_path, grad_y and the per-token gradients) and M0, grad_M_T, grad_M0
 * 16 bytes; lambda0, grad_lambda_T, grad_lambda0 4 bytes.  The workspace holds
 * no flags, so it needs no initialisation.
 * Arithmetic: float32 throughout; dtype outputs are rounded once at the end
 * (bf16: nearest even).  Results are deterministic (fixed summation order).
 */
int kla_backward(const void* q, const void* k, const void* v,
                 const void* log_decay, const void* proc_noise, const void* val_prec,
                 const float* lambda0, const float* M0, const float* lambda_path,
                 const void* grad_y, const float* grad_lambda_T, const float* grad_M_T,
                 void* grad_q, void* grad_k, void* grad_v,
                 void* grad_log_decay, void* grad_proc_noise, void* grad_val_prec,
                 float* grad_lambda0, float* grad_M0,
                 int B, int H, int T, int dk, int dv, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Zero-fills a workspace on `stream` (a fill kernel, no memset node), once
 * before its first use.  bytes must be a multiple of 4. */
int kla_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Reads the device-side error word of a workspace, ordered after the work
 * queued on `stream` (an asynchronous copy on that stream, then a stream
 * synchronisation): 0 = no error; 1 = the outputs of some call are
 * unspecified, because
 *   - a workgroup gave up waiting for a predecessor's carry after about 2^25
 *     polls (1-2 s) and went on with whatever carry it had found, or
 *   - (kla_forward with bf16 inputs at dk = dv = 64) a stretch of tokens
 *     dropped the posterior mean entering it where its decay since the
 *     stretch's start had fallen below 2^-100, and that mean then turned
 *     out to be 2^40 or more in magnitude, so the dropped term may matter.
 * The word is sticky: it stays set for later calls on the same workspace
 * until kla_workspace_init clears it.  The Python binding reads it when a
 * call asks for `check=True`. */
int kla_workspace_error(const void* workspace, int* error_out, void* stream);

/* Static text for a status code; for KLA_ERR_HIP, the last HIP error text
 * recorded on the calling thread. */
const char* kla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KLA_H_ */
