/*
 * dn.h -- C ABI of the chunkwise (gated) delta-rule library for AMD MI355X
 * (gfx950).  All device code behind these calls is hand-written HIP.
 *
 * The operation (Gated DeltaNet review thread, "Gated Delta Networks:
 * Improving Mamba2 with Delta Rule", Table 1, rows "DeltaNet" and
 * "Gated DeltaNet"), per sequence and head, token by token:
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with S_t in R^{Dv x Dk}, alpha_t = exp(g_t) (alpha == 1 without a gate) and
 * no query scaling.  The library evaluates it chunkwise: 64-token chunks whose
 * products of Householder-like transitions are written in WY/UT form
 * ("Parallelizing Linear Transformers with the Delta Rule over Sequence
 * Length", page 3 abstract, and page 1 answers Q1/Q2), which is exact: results
 * differ from the token loop only by floating-point rounding.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *   never allocates, frees, or synchronises; each call enqueues its kernels on
 *   `stream` and returns.  Inputs are read-only (except the decode `state`
 *   and dn_longhorn_eps_bwd's `dk`, updated in place).  There is no global mutable state: calls are
 *   thread-safe; calls sharing a workspace on different streams race.
 * - Layouts are dense row-major:
 *     q, k        [B, T, H, Dk]       v, o, dO    [B, T, H, Dv]
 *     beta, g     [B, T, H]  fp32
 *     h0, hT, dhT, dh0   [N, H, Dk, Dv]  fp32, holding h = S^T
 *   N is the number of sequences: B, or n_seqs when `cu_seqlens` is given.
 * - Packed variable-length input: `cu_seqlens` (device, int32 [n_seqs + 1],
 *   non-decreasing, cu[0] = 0, cu[n_seqs] = T) requires B == 1; sequence n
 *   covers tokens [cu[n], cu[n+1]) and chunks restart at every sequence start.
 *   A zero-length sequence passes its h0 through to hT.  The library does not
 *   copy cu_seqlens to the host; malformed offsets are undefined behaviour.
 *   The sequential passes take packed sequences longest first: a small kernel
 *   ranks them by length into the workspace, so that the longest sequence,
 *   whose chain of chunks is the critical path, starts in the first wave of
 *   workgroups wherever it sits in the pack (packs of more than 65536
 *   sequences keep their own order).  The results do not depend on it.
 * - Validation happens on the host before any launch; on error nothing is
 *   enqueued.  Kernel faults surface at the caller's next synchronisation.
 * - Supported: Dk in {64, 128}; Dv a positive multiple of 64 up to 1024;
 *   chunk == 64, or 32 for DN_BF16 inputs in dn_chunk_fwd, dn_chunk_fwd_save,
 *   dn_chunk_bwd, dn_chunk_bwd_events, dn_chunk_bwd_saved and
 *   dn_chunk_bwd_noalloc (the same result with 32-token chunks: the chunk
 *   form is an exact refactoring of the token recurrence; the backward
 *   workspace then holds twice the chunk states); dtype DN_BF16, or DN_F32
 *   in dn_chunk_fwd with Dk == 64 and in dn_recurrent_step (q, k, v, o, dO
 *   share it; every pass that uses the backward workspace is bf16 only); all
 *   pointers 16-byte aligned; 256 H max(Dk, Dv) < 2^31 (the byte span of one
 *   64-token chunk of fp32 rows, addressed with 32-bit offsets); for the
 *   backward passes, fewer than 2^31 (chunk, head) pairs.  Shapes outside
 *   these limits return DN_EUNSUPPORTED.
 */
#ifndef DN_H_
#define DN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DN_OK = 0,
    DN_EINVAL = 1,       /* null required pointer, bad dims, misalignment, g/dg mismatch */
    DN_EUNSUPPORTED = 2, /* valid but not implemented: Dk, Dv, chunk, dtype            */
    DN_ENOWS = 3,        /* workspace smaller than the query function's answer          */
    DN_EHIP = 4,         /* a HIP launch reported an error                              */
    DN_ESCRATCH = 5      /* dn_chunk_bwd_noalloc: the shape exceeds its static scratch  */
} dn_status;

typedef enum { DN_F32 = 0, DN_BF16 = 1 } dn_dtype;

/* Problem shape.  For packed input B == 1, T is the total token count and
 * n_seqs the number of sequences; otherwise n_seqs must equal B. */
typedef struct {
    int32_t B, T, H, Dk, Dv;
    int32_t n_seqs;
    int32_t chunk;   /* chunk length: 64 (32 also for bf16 inputs, see above) */
    int32_t dtype;   /* dn_dtype of q, k, v, o, dO */
} dn_shape;

/* Human-readable name of a status code (static string). */
const char *dn_status_str(dn_status s);

/* Bytes of device workspace dn_chunk_fwd needs for this shape: for packed
 * input (the query assumes it when B == 1 or n_seqs != B) 4 bytes per
 * sequence, rounded up to 256, for the order in which the pass takes the
 * sequences; 0 otherwise (then workspace may be NULL). */
size_t dn_chunk_fwd_workspace(const dn_shape *s);

/*
 * Chunkwise forward pass.  Produces o for every token and, if hT != NULL, the
 * final state of every (sequence, head).  g == NULL means no gate (alpha = 1);
 * h0 == NULL means a zero initial state.  The per-chunk WY/UT factors and the
 * chunk-start states stay on chip; nothing but o and hT is written
 * (Parallelizing Linear Transformers..., page 1, answer Q2, describes the
 * materialise-then-recompute trade-off this pass avoids for inference).
 * With cu_seqlens the workspace (16-byte aligned) must hold
 * dn_chunk_fwd_workspace(s) bytes (DN_ENOWS otherwise); the call writes the
 * sequence order there.
 */
dn_status dn_chunk_fwd(const dn_shape *s,
                       const void *q, const void *k, const void *v,
                       const float *beta, const float *g, const float *h0,
                       const int32_t *cu_seqlens,
                       void *o, float *hT,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace dn_chunk_bwd needs for this shape. */
size_t dn_chunk_bwd_workspace(const dn_shape *s);

/*
 * Chunkwise backward pass of L = <dO, o> + <dhT, hT> (dhT == NULL means 0).
 * Recomputes the chunk-start states in a forward sweep (the recompute-in-the-
 * backward design of Parallelizing Linear Transformers..., page 1, answer Q2),
 * then runs a reverse sweep for the state gradients and a chunk-parallel pass
 * for the token gradients.  Writes fp32 gradients in the input layouts:
 * dq, dk [B,T,H,Dk], dv [B,T,H,Dv], dbeta [B,T,H], dg [B,T,H] (must be NULL
 * exactly when g is NULL), dh0 [N,H,Dk,Dv] (NULL skips it).  bf16 inputs
 * only (DN_EUNSUPPORTED for DN_F32).
 */
dn_status dn_chunk_bwd(const dn_shape *s,
                       const void *q, const void *k, const void *v,
                       const float *beta, const float *g, const float *h0,
                       const int32_t *cu_seqlens,
                       const void *dO, const float *dhT,
                       float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dn_chunk_bwd with stage timing: the same operation, arguments and errors,
 * and in addition it records events[0] on `stream` before its first kernel,
 * events[1] after the state recompute, events[2] after the reverse
 * state-gradient sweep and events[3] after the chunk-gradient kernel (whose
 * launch follows the sweep directly), so that hipEventElapsedTime on
 * consecutive pairs gives each stage's device time.  The four events are
 * created (with timing enabled) and owned by the caller; a NULL entry is
 * not recorded, and events == NULL is dn_chunk_bwd.  A failed record returns
 * DN_EHIP.
 */
dn_status dn_chunk_bwd_events(const dn_shape *s,
                              const void *q, const void *k, const void *v,
                              const float *beta, const float *g, const float *h0,
                              const int32_t *cu_seqlens,
                              const void *dO, const float *dhT,
                              float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                              void *workspace, size_t workspace_bytes, hipStream_t stream,
                              hipEvent_t *events);

/*
 * Training forward pass that keeps the chunk states for the backward pass
 * (the materialising alternative of Parallelizing Linear Transformers...,
 * page 1, answer Q2: chunk-level states written to HBM in the forward pass,
 * so that the backward pass need not recompute them).  The same operation,
 * arguments, outputs and errors as dn_chunk_fwd, bf16 only
 * (DN_EUNSUPPORTED otherwise), and in addition it writes every chunk-start
 * state S = h^T in bf16 (and, for packed input, the chunk table) into
 * `workspace`, which must hold dn_chunk_bwd_workspace(s) bytes
 * (DN_ENOWS otherwise).  The workspace then belongs to the matching
 * dn_chunk_bwd_saved call; its contents are opaque.
 */
dn_status dn_chunk_fwd_save(const dn_shape *s,
                            const void *q, const void *k, const void *v,
                            const float *beta, const float *g, const float *h0,
                            const int32_t *cu_seqlens,
                            void *o, float *hT,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass from saved states: dn_chunk_bwd_events without the state
 * recompute.  It reads the chunk-start states that dn_chunk_fwd_save stored
 * in `workspace`; the caller guarantees that q, k, v, beta, g, h0,
 * cu_seqlens and the workspace are unchanged since that call and that the
 * call is ordered after it (same stream, or synchronised); otherwise the
 * gradients are those of whatever states the workspace holds.  Arguments,
 * outputs and errors as dn_chunk_bwd_events; events (NULL: none) are recorded
 * as there, events[0] and events[1] back to back since there is no recompute.
 */
dn_status dn_chunk_bwd_saved(const dn_shape *s,
                             const void *q, const void *k, const void *v,
                             const float *beta, const float *g, const float *h0,
                             const int32_t *cu_seqlens,
                             const void *dO, const float *dhT,
                             float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                             void *workspace, size_t workspace_bytes, hipStream_t stream,
                             hipEvent_t *events);

/*
 * dn_chunk_bwd_saved with the input prologue's backward folded in: for inputs
 * that dn_prologue prepared (q = q_in / |q_in|, k = k_in / |k_in|,
 * beta = sigmoid(b_in), g = -gate_scale softplus(x_in)), writes the gradients
 * of L with respect to the raw inputs instead of those of q, k, beta, g:
 * dq_in, dk_in [B,T,H,Dk], db_in, dx_in [B,T,H] (fp32; dx_in NULL exactly when
 * g and x_in are NULL), plus dv and dh0 as dn_chunk_bwd_saved.  The same values
 * as dn_chunk_bwd_saved followed by dn_prologue_bwd, up to summation order,
 * without the fp32 dq, dk, dbeta, dg round trip through HBM.  q, k, beta, g are
 * the prologue's outputs (the recurrence's inputs), q_in and k_in (dtype of q)
 * its raw inputs; the workspace is the one dn_chunk_fwd_save filled.  Errors as
 * dn_chunk_bwd_saved, DN_EINVAL for null or misaligned q_in, k_in (T > 0)
 * or an x_in/g nullness mismatch, and DN_EUNSUPPORTED for chunk == 32 (this
 * variant runs 64-token chunks only).
 */
dn_status dn_chunk_bwd_prologue(const dn_shape *s,
                                const void *q, const void *k, const void *v,
                                const float *beta, const float *g, const float *h0,
                                const int32_t *cu_seqlens,
                                const void *dO, const float *dhT,
                                const void *q_in, const void *k_in, const float *x_in, float gate_scale,
                                float *dq_in, float *dk_in, float *dv, float *db_in, float *dx_in,
                                float *dh0,
                                void *workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t *events);

/*
 * dn_chunk_bwd_saved for the Longhorn recurrence, with the step size's
 * backward folded in: the recurrence ran at beta := eps = beta / (1 + beta
 * |k|^2) (dn_longhorn_eps; Gated DeltaNet review thread, Table 1, row
 * "Longhorn"), `eps` is that step size and `beta` the raw one.  Writes dq,
 * dv, dg, dh0 as dn_chunk_bwd_saved, dk with the step size's key term
 * -2 eps^2 deps k added, and dbeta, the gradient of the raw beta,
 * deps / (1 + beta |k|^2)^2.  The same values as dn_chunk_bwd_saved followed
 * by dn_longhorn_eps_bwd up to rounding (here (eps / beta)^2 stands for
 * 1 / (1 + beta |k|^2)^2).  The workspace is the one dn_chunk_fwd_save filled
 * with beta := eps.  Errors as dn_chunk_bwd_saved, DN_EINVAL for a null
 * beta (T > 0), and DN_EUNSUPPORTED for chunk == 32 (64-token chunks only).
 */
dn_status dn_chunk_bwd_longhorn(const dn_shape *s,
                                const void *q, const void *k, const void *v,
                                const float *eps, const float *g, const float *h0,
                                const int32_t *cu_seqlens,
                                const void *dO, const float *dhT,
                                const float *beta,
                                float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                                void *workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t *events);

/*
 * dn_chunk_bwd_noalloc -- dn_chunk_bwd (the recomputing backward pass, same
 * kernels, same results bit for bit) for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace: its chunk states, state
 * gradients and packed-sequence chunk table live in a static device buffer
 * of DN_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU it
 * runs on until the process ends.  The call itself allocates nothing; the
 * buffer's address on the current device is looked up once, on the first
 * call on that device.  The shape may need at most that many workspace bytes
 * (dn_chunk_bwd_workspace(s) <= DN_NOALLOC_SCRATCH_BYTES; B 1, T 2048,
 * H 16, Dk 128, Dv 128 needs 34.6 MB); a larger one returns DN_ESCRATCH
 * before anything is enqueued.  Every call on one GPU shares that GPU's buffer:
 * calls that overlap in time on one GPU (different streams, or different
 * host threads) race and give wrong results; calls on one stream are
 * ordered and safe.  Nothing in the buffer needs clearing between calls
 * (every byte a call reads it first writes).  Arguments, layouts and the
 * other errors are those of dn_chunk_bwd.
 */
#define DN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dn_status dn_chunk_bwd_noalloc(const dn_shape *s,
    const void *q, const void *k, const void *v, const float *beta, const float *g,
    const float *h0, const int32_t *cu_seqlens, const void *dO, const float *dhT,
    float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dh0,
    hipStream_t stream);

/*
 * One recurrent (decode) step for B x H independent states: the token update
 * above applied once (Gated DeltaNet review thread, General Response 2: the
 * recurrent step is memory-bound and its cost is set by the state size).
 * q, k [B,H,Dk]; v, o [B,H,Dv] (dtype); beta, g [B,H] fp32 (g may be NULL);
 * state [B,H,Dk,Dv] fp32 holding S^T, read and overwritten in place.
 * Supported: Dk in {64, 128}, Dv a positive multiple of 64 up to 1024.
 */
dn_status dn_recurrent_step(int32_t B, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                            const void *q, const void *k, const void *v,
                            const float *beta, const float *g,
                            float *state, void *o, hipStream_t stream);

/*
 * Longhorn step size (Gated DeltaNet review thread, Table 1, row "Longhorn",
 * with the caption's scalar beta): the Longhorn recurrence is the delta rule
 * with beta_t replaced by
 *
 *     eps_t = beta_t / (1 + beta_t k_t^T k_t),
 *
 * so it runs as dn_longhorn_eps followed by dn_chunk_fwd / dn_recurrent_step
 * with beta := eps.  The table's row has no decay; a gate g given to those
 * calls still multiplies the state.
 * k [B,T,H,Dk] (dtype, for decode T = 1), beta and eps [B,T,H] fp32; rows are
 * independent.  Supported: Dk in {64, 128}; k 16-byte aligned.  T == 0 is a
 * no-op.  Nothing is allocated; the call enqueues one kernel on `stream`.
 */
dn_status dn_longhorn_eps(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype,
                          const void *k, const float *beta, float *eps, hipStream_t stream);

/*
 * Backward of dn_longhorn_eps (the chain rule through eps; s = k^T k):
 *
 *     dbeta = deps / (1 + beta s)^2
 *     dk   += deps * (-2 beta^2 / (1 + beta s)^2) * k
 *
 * deps is the beta-gradient that dn_chunk_bwd returns when it is called with
 * beta := eps; dk [B,T,H,Dk] fp32 (16-byte aligned) is the key gradient of
 * that call and is updated in place.  dbeta may alias deps.
 */
dn_status dn_longhorn_eps_bwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype,
                              const void *k, const float *beta, const float *deps,
                              float *dbeta, float *dk, hipStream_t stream);

/*
 * Input prologue of a (Gated) DeltaNet layer: the preparation applied to the
 * projections before the recurrence, one fused pass per (token, head) row.
 * The pages name the layer's parts around the token mixer (the DeltaNet
 * rebuttal, answer W2: depthwise short convolutions; Table 1: beta, alpha)
 * but give no formula; this is the preparation the workloads use:
 *
 *     q = q_in / |q_in|,  k = k_in / |k_in|     (a zero row stays zero)
 *     beta = sigmoid(b_in),  g = -gate_scale * softplus(x_in)
 *
 * q_in, k_in, q, k [B,T,H,Dk] (dtype, 16-byte aligned); b_in, x_in, beta, g
 * [B,T,H] fp32.  x_in == NULL (then g must be NULL too) means no gate.
 * Supported: Dk in {64, 128}.  T == 0 is a no-op.  The short convolution is
 * not part of this call.
 */
dn_status dn_prologue(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype,
                      const void *q_in, const void *k_in, const float *b_in, const float *x_in,
                      float gate_scale, void *q, void *k, float *beta, float *g,
                      hipStream_t stream);

/*
 * Backward of dn_prologue: from the gradients w.r.t. its outputs (dq, dk
 * [B,T,H,Dk] fp32 as dn_chunk_bwd returns them; dbeta, dg [B,T,H] fp32) to
 * those of its inputs, all fp32:
 *
 *     dq_in = (dq - q (q . dq)) / |q_in|   (likewise dk_in; 0 for a zero row)
 *     db_in = dbeta * beta * (1 - beta),   dx_in = -gate_scale * sigmoid(x_in) * dg
 *
 * x_in, dg and dx_in are all NULL or all given.  Outputs may not alias inputs.
 */
dn_status dn_prologue_bwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype,
                          const void *q_in, const void *k_in, const float *b_in,
                          const float *x_in, float gate_scale,
                          const float *dq, const float *dk, const float *dbeta, const float *dg,
                          float *dq_in, float *dk_in, float *db_in, float *dx_in,
                          hipStream_t stream);

/*
 * Depthwise causal short convolution (the DeltaNet rebuttal, answer W2: the
 * "short convolution" layers the layer applies beside the token mixer, here
 * to any [B,T,H,D] projection).  Every channel (h, c) has its own W taps and
 * a token sees itself and the W - 1 tokens before it in its own sequence:
 *
 *     y[t, h, c] = sum_{j < W} w[h, c, j] x[t - (W - 1) + j, h, c]
 *
 * with x = 0 before the sequence's first token (tap W - 1 is the current
 * token).  The pages give neither the width nor an activation: the width is
 * the caller's (1 to 4) and no activation is applied.  x, y [B,T,H,D] (dtype,
 * 16-byte aligned; y may not alias x); w [H,D,W] fp32.  Packed sequences:
 * cu_seqlens (device int32 [n_seqs + 1], as dn_chunk_fwd) with B == 1;
 * otherwise cu_seqlens NULL and n_seqs == B.  T == 0 is a no-op.
 * DN_EINVAL for bad sizes, dtype, null or misaligned pointers;
 * DN_EUNSUPPORTED for D not a multiple of 8 or W outside 1..4.
 */
dn_status dn_short_conv(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                        int32_t dtype, const void *x, const float *w, const int32_t *cu_seqlens,
                        void *y, hipStream_t stream);

/*
 * Backward of dn_short_conv, from dy = dL/dy [B,T,H,D] fp32:
 *
 *     dx[p, h, c] = sum_{j < W} w[h, c, j] dy[p + (W - 1) - j, h, c]   (outputs of p's sequence)
 *     dw[h, c, j] = sum_p x[p, h, c] dy[p + (W - 1) - j, h, c]
 *
 * dx [B,T,H,D] fp32 (16-byte aligned), dw [H,D,W] fp32, both overwritten (dw
 * is cleared on the stream first, then accumulated with atomic adds, so its
 * summation order may differ between calls; with T == 0 it is set to zero);
 * neither may alias an input.  Other arguments and errors as dn_short_conv.
 */
dn_status dn_short_conv_bwd(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                            int32_t dtype, const void *x, const float *w, const int32_t *cu_seqlens,
                            const float *dy, float *dx, float *dw, hipStream_t stream);

/*
 * dn_short_conv fused with the L2 normalisation of dn_prologue: every
 * (token, head) row of the convolution's output z is scaled to unit length,
 *
 *     y[t, h, :] = z[t, h, :] / |z[t, h, :]|     (a zero row stays zero)
 *
 * in the same pass, which is how a (Gated) DeltaNet layer prepares q and k
 * from their projections (the rebuttal's short convolutions, then the
 * workloads' normalisation).  D in {64, 128}; otherwise as dn_short_conv.
 */
dn_status dn_short_conv_l2(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                           int32_t dtype, const void *x, const float *w, const int32_t *cu_seqlens,
                           void *y, hipStream_t stream);

/*
 * Backward of dn_short_conv_l2 from dy = dL/dy (fp32): z is recomputed from x
 * and w, dz = (dy - u (u . dy)) / |z| with u = z / |z| (0 for a zero row),
 * then dx and dw are those of dn_short_conv_bwd for dz.  Arguments, output
 * semantics (dw cleared, then accumulated atomically) and errors as
 * dn_short_conv_bwd; D in {64, 128}.
 */
dn_status dn_short_conv_l2_bwd(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                               int32_t dtype, const void *x, const float *w, const int32_t *cu_seqlens,
                               const float *dy, float *dx, float *dw, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DN_H_ */
