/*
 * s6.h -- C ABI of libs6, the selective-SSM scan (S6) library for AMD MI355X
 * (gfx950).
 *
 * The operation.  Sources: the page "【LLM】Mamba和State Space Models详解" (a
 * Chinese translation of a visual guide to Mamba and state space models):
 *   §2.2  continuous SSM h'(t) = A h(t) + B x(t), y(t) = C h(t) + D x(t);
 *         D is a skip connection.
 *   §2.3  zero-order-hold discretisation with a learnable step Delta; the
 *         continuous A is kept and discretised on the fly.  (The formula
 *         image is missing; this library uses dA = exp(Delta*A[d,n]) and
 *         dBx = Delta*B[n]*x.)
 *   §2.4  recurrent form: h_k = dA h_{k-1} + dB x_k, then y_k = C h_k (the
 *         output is read from the updated state).
 *   §3.2  selection: Delta (batch, D, L), B and C (batch, N, L) vary per
 *         token; A (D, N) does not.
 *   §3.3  the scan over time, evaluated with associativity; §3.4 fusion of
 *         discretisation, scan and the product with C in one pass that
 *         never writes the (batch, D, L, N) state to memory.
 * The news page on the Mamba paper ("屹立不倒的 Transformer 迎來了一個強勁競爭者",
 * sections 選擇機制 and 架構) notes that a recurrent model with a finite state
 * needs constant time per generated token: s6_state_update is that step.
 * The optional output gate y <- y * SiLU(z), SiLU(z) = z / (1 + e^-z), is
 * applied after the skip term; it is not drawn on the pages and is the plain
 * reading of the gated Mamba output.
 *
 * Per (batch b, channel d, state n), for t = 0 .. L-1:
 *   h[n]   = exp(delta[b,d,t] * A[d,n]) * h[n] + delta[b,d,t] * Bm[b,n,t] * x[b,d,t]
 *   y[b,d,t] = (sum_n Cm[b,n,t] * h[n] + Dskip[d] * x[b,d,t]) * SiLU(z[b,d,t])
 * starting from h = h0[b,d,:] (or 0); h_last[b,d,:] is h after token L-1.
 *
 * Conventions shared by every entry point
 *   Layout: contiguous row-major, last index fastest.
 *     x, delta, z, y : (batch, dim, seqlen)     Bm, Cm : (batch, dstate, seqlen)
 *     A : (dim, dstate)   Dskip : (dim)          h0, h_last, h : (batch, dim, dstate)
 *     decode step: x, delta, z, y : (batch, dim); Bm, Cm : (batch, dstate)
 *   in_dtype: S6_F32 or S6_BF16; it applies to x, delta, Bm, Cm and z.  A,
 *     Dskip, h0, h, h_last and y are always fp32; the state is fp32.
 *   Pointers: device memory owned by the caller (for example torch
 *     allocations), aligned to their element size; 16-byte alignment and a
 *     seqlen that is a multiple of 8 select the vectorised load path.
 *     Outputs must not alias inputs (except h, updated in place by
 *     s6_state_update).
 *   stream: a hipStream_t passed as void*; NULL is the default stream.  Every
 *     call only enqueues work and returns; the caller synchronises.
 *   Sizes: batch, dim, seqlen >= 0 (zero means no work; with seqlen == 0,
 *     h_last receives h0 or zeros), 1 <= dstate <= 32, and
 *     batch*dim*max(seqlen,1)*max(dstate,...) must fit in int64.
 *   Errors: 0 (S6_OK) or a negative S6_ERR_* code.  All argument checks run
 *     before any HIP call, so a rejected call has no side effect.  Values are
 *     not checked: NaN/Inf propagate.  Accuracy is specified for A <= 0 and
 *     delta >= 0 (decaying states).
 *   Memory: the library allocates nothing and keeps no state between calls
 *     (except s6_scan_fwd_noalloc's static buffer, see there).
 *     Entry points that may need scratch memory take a caller-owned device
 *     workspace (void* workspace, size_t workspace_bytes), 256-byte aligned,
 *     of at least the size the matching *_workspace_size query returns for
 *     the same sizes on the same device (0 when none is needed; NULL is then
 *     accepted).  The forward and final-state scans need one only when there
 *     are too few (batch, channel) blocks to fill the GPU and the sequence is
 *     cut into segments (per-segment carries); the backward always does
 *     (segment states, partial sums).  A call only enqueues work that uses the
 *     workspace: it must stay allocated, and not be used by other work, until
 *     that work has run on the stream.  Too small or NULL when needed:
 *     S6_ERR_WORKSPACE, before any work is enqueued.  Its contents on entry
 *     do not matter and are left undefined.
 */
#ifndef S6_H_
#define S6_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define S6_F32 0
#define S6_BF16 1

#define S6_OK 0
#define S6_ERR_NULL (-1)        /* a required pointer is NULL */
#define S6_ERR_SHAPE (-2)       /* a size is negative or the element count overflows */
#define S6_ERR_DTYPE (-3)       /* in_dtype is not S6_F32 or S6_BF16 */
#define S6_ERR_UNSUPPORTED (-4) /* dstate outside 1..32, a filter width outside 1..4, or an option the entry point lacks */
#define S6_ERR_ALIGN (-5)       /* a pointer is not aligned to its element size */
#define S6_ERR_HIP (-6)         /* a HIP call failed; s6_status_str gives the detail */
#define S6_ERR_FLAGS (-7)       /* unknown bits in the flags of an _ex entry point */
#define S6_ERR_WORKSPACE (-8)   /* the workspace is NULL or smaller than its *_workspace_size */

/* Options of the _ex entry points (bit flags). */
#define S6_DELTA_SOFTPLUS 1 /* step = softplus(delta + delta_bias[d]) */
#define S6_ZOH_EXACT 2      /* input term (exp(step*A) - 1) / A * B * x */

/* Version of this ABI, major*10000 + minor*100 + patch. */
int s6_version(void);

/* Human-readable text for a status code.  For S6_ERR_HIP it includes the
 * last HIP error seen by this thread.  The string is static or thread-local. */
const char* s6_status_str(int status);

/* Fused selective scan: discretisation, recurrence over the whole sequence,
 * contraction with C, skip term and optional gate, in one pass that keeps
 * the state on chip.
 *   x, delta, Bm, Cm, A : required.
 *   Dskip : nullable (no skip term).    z : nullable (no gate).
 *   h0    : nullable (zero initial state).
 *   y     : required output (batch, dim, seqlen) fp32.
 *   h_last: nullable output (batch, dim, dstate) fp32, the state after the
 *           last token.
 *   workspace, workspace_bytes: see Memory above; the size is
 *           s6_scan_fwd_workspace_size for the same sizes (it serves the
 *           _ex, _ckpt and convolution-front forms as well). */
int s6_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* h0, float* y, float* h_last,
                void* workspace, size_t workspace_bytes, void* stream);

/* s6_scan_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; when the sequence is cut into segments, their
 * carries go to a static device buffer of the library (16 MiB, one per GPU,
 * held until the process ends; its address is looked up once per device on
 * the first call there).  No hipMalloc, hipFree or allocating library call.
 * A call that would need more than 16 MiB returns S6_ERR_WORKSPACE before any
 * work is enqueued (on a 256-CU device a segmented forward needs at most
 * about 6 MB, whatever the sequence length).  Every call on one GPU shares
 * that buffer and leaves its contents behind (nothing in it needs to start
 * at zero): calls that overlap on one GPU -- concurrent streams, or host
 * threads -- race and must be serialised by the caller.  Same arguments,
 * checks and results as s6_scan_fwd otherwise. */
int s6_scan_fwd_noalloc(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                        const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                        const float* Dskip, const void* z, const float* h0, float* y, float* h_last,
                        void* stream);

/* Workspace size in bytes (*bytes) of the forward scans (s6_scan_fwd,
 * s6_scan_fwd_ex, s6_scan_fwd_ckpt, s6_conv_scan_fwd) and of the final-state
 * scans (s6_last_state, s6_last_state_ex) for these sizes on the current
 * device.  Checks the sizes as the entry points do; bytes: required. */
int s6_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                               size_t* bytes);
int s6_last_state_workspace_size(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                                 size_t* bytes);

/* Final state only (prefill -> decode hand-off, or a sequence shard's
 * carry): the recurrence of s6_scan_fwd without C, D, z or y.
 *   h0 : nullable.   h_last : required output (batch, dim, dstate) fp32.
 *   workspace: s6_last_state_workspace_size bytes. */
int s6_last_state(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                  const void* x, const void* delta, const float* A, const void* Bm,
                  const float* h0, float* h_last, void* workspace, size_t workspace_bytes, void* stream);

/* One decode token for every (batch, channel): h is read, advanced by one
 * step and written back in place; y receives the token's output.  batch*dim
 * above 2^31 * 32 is rejected with S6_ERR_SHAPE (launch grid limit).
 *   h : required, in/out (batch, dim, dstate) fp32.
 *   x, delta, z : (batch, dim); Bm, Cm : (batch, dstate); Dskip and z nullable.
 *   y : required output (batch, dim) fp32. */
int s6_state_update(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                    const void* x, const void* delta, const float* A, const void* Bm,
                    const void* Cm, const float* Dskip, const void* z, float* y, void* stream);

/* The same three operations with a per-channel step bias and the
 * discretisation options.  §3.2 of the guide makes Delta learned and
 * input-dependent without saying how it stays positive, and §2.3 names the
 * zero-order hold without its formula (the image is missing):
 *   delta_bias : nullable (dim) fp32; the step is delta[b,d,t] + delta_bias[d].
 *   S6_DELTA_SOFTPLUS : the step is softplus(delta + delta_bias[d]),
 *       softplus(v) = ln(1 + e^v), computed in fp32 as the delta tile is
 *       staged.
 *   S6_ZOH_EXACT : the input term is held over the step as well as the
 *       state: h[n] = exp(s*A[d,n]) * h[n] + (exp(s*A[d,n]) - 1) / A[d,n] *
 *       Bm[b,n,t] * x[b,d,t] for the step s (s * Bm * x where A[d,n] = 0),
 *       instead of s * Bm * x.
 * flags = 0 and delta_bias = NULL give exactly s6_scan_fwd, s6_last_state
 * and s6_state_update.  Other flag bits: S6_ERR_FLAGS.  delta_bias must be
 * 4-byte aligned.  Everything else is as for the plain entry points. */
int s6_scan_fwd_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                   const void* x, const void* delta, const float* delta_bias, int flags,
                   const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                   const float* h0, float* y, float* h_last, void* workspace, size_t workspace_bytes,
                   void* stream);

int s6_last_state_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const float* h0, float* h_last, void* workspace,
                     size_t workspace_bytes, void* stream);

int s6_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                       const void* x, const void* delta, const float* delta_bias, int flags,
                       const float* A, const void* Bm, const void* Cm, const float* Dskip,
                       const void* z, float* y, void* stream);

/* The scan with the convolution front of the Mamba block.  §3.5 of the
 * guide ("Mamba Block") applies a convolution to the expanded input before
 * the selective SSM, so that tokens are not handled independently; it gives
 * neither the width nor an activation.  Here: per channel a causal filter of
 * conv_width taps and a bias, then SiLU, and the scan (with its skip term)
 * takes the result as its input x:
 *   x'[b,d,t] = SiLU(conv_bias[d] + sum_{k<K} conv_w[d,k] * x[b,d,t-K+1+k]),
 * K = conv_width, where inputs before token 0 are conv_state[b,d,K-1+s] for
 * s = -(K-1) .. -1 (oldest first), or 0 when conv_state is NULL.  The
 * filtered input is computed in fp32 as x is staged and never written.
 *   conv_w     : required (dim, conv_width) fp32.  conv_width: 1..4, else
 *                S6_ERR_UNSUPPORTED.
 *   conv_bias  : nullable (dim) fp32.   conv_state : nullable (batch, dim,
 *                conv_width - 1) fp32.  All three 4-byte aligned.
 * The last conv_width - 1 inputs of a sequence (the state of its
 * continuation) are x itself: the caller keeps them.  Everything else is as
 * for s6_scan_fwd_ex (step bias, S6_DELTA_SOFTPLUS, S6_ZOH_EXACT). */
int s6_conv_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const float* conv_w, const float* conv_bias, int conv_width,
                     const float* conv_state, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                     const float* h0, float* y, float* h_last, void* workspace, size_t workspace_bytes,
                     void* stream);

/* One decode token with the convolution front of s6_conv_scan_fwd: the
 * filter runs over the conv_width - 1 kept inputs and this token's x, the
 * scan step takes SiLU of the result as its input, and the kept inputs move
 * on by one (the oldest dropped, x appended):
 *   conv_state : (batch, dim, conv_width - 1) fp32, in/out, oldest first;
 *                required when conv_width > 1.
 * A sequence scanned by s6_conv_scan_fwd continues here with conv_state =
 * its last conv_width - 1 inputs and h = its h_last.  Everything else is as
 * for s6_state_update_ex. */
int s6_conv_state_update(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                         float* conv_state, const void* x, const float* conv_w, const float* conv_bias,
                         int conv_width, const void* delta, const float* delta_bias, int flags,
                         const float* A, const void* Bm, const void* Cm, const float* Dskip,
                         const void* z, float* y, void* stream);

/* Gradients of the scan (reverse mode) for the loss <dy, y> + <dh_last,
 * h_last>, plain step (no options), same inputs as s6_scan_fwd.  The guide's
 * §3.4 notes that the fused scan recomputes the states in the backward pass
 * rather than storing them: the states entering every 64-token segment are
 * recomputed by a state-only pass and the carry fold, and each segment's
 * states again in registers while the adjoint
 *   lambda_t[n] = dy_t SiLU(z_t) Cm[b,n,t] + exp(delta_{t+1} A[d,n]) lambda_{t+1}[n]
 * runs from the last token back.  All gradients are fp32 and overwrite their
 * buffers:
 *   dy      : required (batch, dim, seqlen) fp32.   dh_last : nullable (zero).
 *   dx, ddelta : required (batch, dim, seqlen).     dz : nullable; written only
 *            when z is given.
 *   dA : required (dim, dstate).  dBm, dCm : required (batch, dstate, seqlen).
 *   dDskip : nullable (dim).   dh0 : nullable (batch, dim, dstate), the
 *            gradient of the initial state (h0 itself may be NULL = zero).
 * Sums over channels (dBm, dCm), over batch rows and tokens (dA, dDskip) are
 * taken in a fixed order: repeated calls give identical bits.
 *   workspace: s6_scan_bwd_workspace_size(..., conv_width = 0, from_ckpt =
 *            0, ...) bytes (see Memory above). */
int s6_scan_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* h0, const float* dy,
                const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm, float* dCm,
                float* dDskip, float* dz, float* dh0, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace size in bytes (*bytes) of the backward entry points on the
 * current device: conv_width = 0 for s6_scan_bwd, s6_scan_bwd_ex and
 * s6_scan_bwd_ckpt, the filter width for s6_conv_scan_bwd; from_ckpt != 0
 * for s6_scan_bwd_ckpt (it needs no room for the recomputed segment
 * states).  Its largest parts are the per-16-channel-block partial sums of
 * dBm and dCm (2 * ceil(dim/16) * batch * dstate * seqlen floats) and, without
 * checkpoints, the recomputed states: where batch * ceil(dim/32) workgroups
 * of a sequential scan fill the GPU, the state entering every 16-token chunk
 * (batch * dim * dstate * ceil(seqlen/16) floats), otherwise that entering
 * every 64-token segment with the segments' end states (about twice
 * batch * dim * dstate * ceil(seqlen/64) floats). */
int s6_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                               int conv_width, int from_ckpt, size_t* bytes);

/* s6_scan_bwd with the step bias and the options of s6_scan_fwd_ex (other
 * flag bits: S6_ERR_FLAGS).  ddelta is then the gradient of the stored delta
 * (the step's gradient times dstep/dv, v = delta + delta_bias[d],
 * 1/(1 + e^-v) under softplus), and ddelta_bias (nullable, (dim) fp32)
 * receives its sum over batch rows and tokens.  With S6_ZOH_EXACT the input
 * term's coefficient c = (exp(s*A) - 1) / A enters the gradients: dx and dBm
 * take c where the plain step has s, ddelta's input part takes dc/ds =
 * exp(s*A), and dA gains the term of dc/dA (a series where |s*A| < 1/2).
 * flags = 0 with both bias pointers NULL is s6_scan_bwd. */
int s6_scan_bwd_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                   const void* x, const void* delta, const float* delta_bias, int flags, const float* A,
                   const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
                   const float* dy, const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm,
                   float* dCm, float* dDskip, float* dz, float* dh0, float* ddelta_bias, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Gradients of s6_conv_scan_fwd: the scan's gradients as from s6_scan_bwd_ex
 * (with the same step options), taken on the filtered input x', then carried
 * back through SiLU and the filter:
 *   dxc_t = dx'_t SiLU'(xc_t)        (xc: the filter's output before SiLU)
 *   dx[b,d,s]         = sum_k conv_w[d,k] dxc_{s+K-1-k}  (terms past the end absent)
 *   dconv_state[b,d,K-1+s] = the same sum for s = -(K-1) .. -1
 *   dconv_w[d,k]      = sum_{b,t} dxc_t x_{t-K+1+k} (inputs before token 0 from
 *                       conv_state, or 0)
 *   dconv_bias[d]     = sum_{b,t} dxc_t
 * x' is recomputed as the forward computes it (never stored).  dconv_w is
 * required (dim, conv_width); dconv_bias (dim) and dconv_state (batch, dim,
 * conv_width - 1) are nullable; every other argument as for s6_scan_bwd_ex
 * and s6_conv_scan_fwd, except that S6_ZOH_EXACT is not taken here
 * (S6_ERR_UNSUPPORTED).  Sums over rows and tokens are taken in a fixed
 * order: repeated calls give identical bits. */
int s6_conv_scan_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const float* conv_w, const float* conv_bias, int conv_width,
                     const float* conv_state, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                     const float* h0, const float* dy, const float* dh_last, float* dx, float* ddelta,
                     float* dA, float* dBm, float* dCm, float* dDskip, float* dz, float* dh0,
                     float* ddelta_bias, float* dconv_w, float* dconv_bias, float* dconv_state, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Checkpoints for training: the forward saves the state entering every
 * S6_CKPT_TOKENS-token block, and the backward starts from them instead of
 * recomputing them.  The pages' guide (§3.4) has the fused scan recompute the
 * intermediate states in the backward pass rather than read them from slow
 * memory; these two entry points keep one state in S6_CKPT_TOKENS from the
 * forward pass (1/64 of the states: 4 * batch * dim * dstate bytes per 64
 * tokens) and still recompute everything inside a block.
 *   ckpt : (ceil(seqlen / S6_CKPT_TOKENS), batch, dim, dstate) fp32; block s
 *          holds the state before token S6_CKPT_TOKENS * s (block 0: h0, or
 *          0).  Written by s6_scan_fwd_ckpt, read by s6_scan_bwd_ckpt;
 *          required (S6_ERR_NULL) when there is any work.  4-byte aligned.
 * s6_scan_fwd_ckpt is s6_scan_fwd_ex plus the checkpoints.  s6_scan_bwd_ckpt
 * is s6_scan_bwd_ex with ckpt in place of h0 (the same inputs and options as
 * the forward that wrote it). */
#define S6_CKPT_TOKENS 64
int s6_scan_fwd_ckpt(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                     const float* h0, float* y, float* h_last, float* ckpt, void* workspace,
                     size_t workspace_bytes, void* stream);

int s6_scan_bwd_ckpt(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const void* delta, const float* delta_bias, int flags, const float* A,
                     const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* ckpt,
                     const float* dy, const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm,
                     float* dCm, float* dDskip, float* dz, float* dh0, float* ddelta_bias, void* workspace,
                     size_t workspace_bytes, void* stream);

/* The scan with one A value per channel, A[d, n] = a_d for every state n,
 * computed in chunked matrix form on the matrix cores.  The paper-list page's
 * Mamba-2 abstract (structured state space duality) observes that a scan with
 * such an A is a structured semiseparable matrix whose blocks are matrix
 * products; the result is the recurrence of s6_scan_fwd (the guide's §2.3,
 * §2.4, §3.2) with A[d, n] = A[d]:
 *   h[n] = exp(delta[b,d,t] * A[d]) * h[n] + delta[b,d,t] * Bm[b,n,t] * x[b,d,t]
 *   y[b,d,t] = (sum_n Cm[b,n,t] * h[n] + Dskip[d] * x[b,d,t]) * SiLU(z[b,d,t])
 * evaluated per 16-token chunk as products with the Gram matrix of B and C
 * (shared by every channel of a batch row) and two exponentials per token
 * and channel.  bf16 inputs: every product runs on the bf16 matrix cores;
 * those of inputs only (B, C, their Gram matrix) are exact, and each fp32
 * operand (the scaled inputs, the state, the decayed Gram matrix) enters as
 * the sum of two bf16 parts, within 2^-17 of its value.  fp32 inputs: every
 * product on the fp32 matrix cores.
 *   A : (dim) fp32, one value per channel (accuracy specified for A <= 0).
 *   dstate : 1..16 (else S6_ERR_UNSUPPORTED).
 *   Everything else (layouts, nullable Dskip, z, h0, h_last; errors; stream)
 *   as for s6_scan_fwd.  workspace: s6_ssd_scan_fwd_workspace_size bytes:
 *   0 when the batch x ceil(dim/16) waves fill the GPU; for few long rows
 *   the sequence is cut into segments (a state-only pass, the carry fold,
 *   the scan of every segment from its incoming state) and the workspace
 *   holds the segments' end states, summed steps and incoming states. */
int s6_ssd_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                    const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                    const float* Dskip, const void* z, const float* h0, float* y, float* h_last,
                    void* workspace, size_t workspace_bytes, void* stream);
int s6_ssd_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                                   size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* S6_H_ */
