/*
 * liblinattn - causal kernelized linear attention on AMD Instinct MI355X
 * (gfx950).  C ABI: plain pointers and sizes only.
 *
 * The operation (sources are web pages, cited by title and section):
 *   - feature map phi: R^d -> R^r; ELU(x)+1 with alpha = 1 ("Choice of phi",
 *     linear-attention-kernel page; "Efficient attention variants" sec. 4) or
 *     Performer FAVOR+ positive random features ("Efficient attention
 *     variants" sec. 6), plus the identity for feeding features directly;
 *   - causal: S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t),
 *     o_t = phi(q_t)^T S_t / phi(q_t)^T z_t with S_0 = 0, z_0 = 0
 *     ("Efficient attention variants" sec. 5; "Recurrent form" of the
 *     linear-attention-kernel page; "Why is linear attention an RNN" of the
 *     linear-attention-and-SSM page).  Token t attends to itself;
 *   - non-causal: S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j),
 *     O = phi(Q) S / phi(Q) z ("Efficient attention variants" sec. 4);
 *   - causal with a fixed per-head decay gamma (RetNet form, "Efficient
 *     attention variants" sec. 7.1): S_t = gamma S_{t-1} + phi(k_t) v_t^T,
 *     z_t = gamma z_{t-1} + phi(k_t), read out normalised as above or, with
 *     normalize = 0, as o_t = phi(q_t)^T S_t (the page's form with the
 *     identity map);
 *   - causal with a per-token scalar gate a_t (the scalar-decay form of
 *     Mamba-2's SSD, "Linear attention and SSM", section on how SSD unifies
 *     SSM and attention: A_t = a_t I, output ((Q K^T) o L) V with
 *     L_ij = a_{j+1} ... a_i): S_t = a_t S_{t-1} + phi(k_t) v_t^T,
 *     z_t = a_t z_{t-1} + phi(k_t), read out as the decay above;
 *   - causal with a gate per token and key channel (GLA form, "Efficient
 *     attention variants" sec. 7.2): S_t = diag(a_t) S_{t-1} + phi(k_t) v_t^T,
 *     z_t = a_t * z_{t-1} + phi(k_t) (elementwise), entry f of a_t keeping
 *     row f of the state, read out as the decay above.
 *
 * Conventions shared by every call
 *   - Tensors are contiguous row-major device buffers owned by the caller:
 *       Q, K [B][H][N][d]; V, O [B][H][N][d_v]; S [B][H][r][d_v]; z [B][H][r];
 *       decode tokens q, k [B][H][d], v, o [B][H][d_v]; omega [r][d].
 *     Every pointer must be 16-byte aligned.
 *   - io_dtype selects the element type of Q, K, V, O, q, k, v, o and X:
 *     LA_F32 (float) or LA_BF16 (bfloat16).  States S, z and the FAVOR+
 *     projection omega are always fp32.  Arithmetic is fp32; bf16 data enter
 *     the matrix cores as bf16 with fp32 accumulation.  Outputs are rounded
 *     to nearest-even.
 *   - r: feature dimension.  For LA_PHI_ELU1 and LA_PHI_IDENTITY r must equal d
 *     (0 is accepted and means d).  For LA_PHI_FAVOR (and
 *     LA_PHI_FAVOR_PRECISE) r is the number of omega rows.
 *   - stream: a hipStream_t (NULL = the default stream).  All work is enqueued
 *     asynchronously on it.  The library allocates no memory at run time
 *     (la_forward_noalloc's scratch is a static device array) and is
 *     re-entrant; what persists between calls is the span override of
 *     la_set_span_tokens (process-wide), a per-device cache of the CU count
 *     and of the scratch array's address, and the last HIP error string
 *     (per thread).
 *   - The library links the HIP runtime by its soname (libamdhip64.so.7).  In a
 *     process that also uses PyTorch, load PyTorch first so that both share
 *     the runtime PyTorch brings (the Python binding does this); otherwise two
 *     HIP runtimes end up in one process.
 *   - The returned status covers argument checks and launch errors
 *     (LA_ERR_HIP after hipGetLastError).  Numerical results are not errors:
 *     a zero denominator, possible only with the identity map, yields IEEE
 *     inf/NaN in that row.
 *   - Supported shapes (others return LA_ERR_UNSUPPORTED):
 *       la_forward: d = d_v in {64, 128} with ELU1/IDENTITY (bf16), d = d_v = 64
 *       (fp32); chunk in {16, 32, 64, 128} (bf16 d = 64), {16, 32, 64} otherwise;
 *       any N >= 0, any B, H >= 0.
 *       la_forward_decay: as la_forward for ELU1/IDENTITY (no FAVOR+).
 *       la_decode_step: d = d_v in {64, 128}; FAVOR+ with r = 256.
 *       la_decode_step_decay: d = d_v in {64, 128}, ELU1/IDENTITY.
 *       la_forward_gated, la_decode_step_gated: as the decay calls.
 *       la_backward: bf16, ELU1/IDENTITY, d = d_v in {64, 128}, chunk 64 (0 means 64).
 *       la_forward_gla: ELU1/IDENTITY, d = d_v = 64 (bf16: chunk 16..128;
 *       fp32: 16..64) or d = d_v = 128 (bf16, chunk 16 or 32; chunk = 0
 *       means 32 there); la_decode_step_gla: as the decay decode.
 *       la_feature_map: ELU1/IDENTITY with d % 8 == 0; FAVOR+ with d in {64, 128},
 *       r = 256.
 */
#ifndef LINATTN_LA_H
#define LINATTN_LA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
  LA_OK = 0,
  LA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  LA_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or too large */
  LA_ERR_UNSUPPORTED = 3, /* valid request outside the supported shapes         */
  LA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                   */
  LA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required            */
  LA_ERR_HIP = 6,         /* the HIP runtime reported an error                  */
  LA_ERR_SCRATCH = 7      /* la_forward_noalloc: the call needs more than its fixed scratch */
} la_status;

typedef enum la_dtype { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Feature maps.  LA_PHI_FAVOR_PRECISE is FAVOR+ with the same features and
 * results up to rounding ("Efficient attention variants", sec. 6); only
 * la_forward's output pass differs: it projects with omega carried as a bf16
 * hi + lo pair instead of bf16 hi, which keeps bf16-level accuracy for inputs
 * whose norms exceed the workloads' (|u| / d^(1/4) of 2 and more, where the
 * fast form's relative error per output row grows to about 1.5e-2 and, at
 * 8, 5e-2), at about 1.45 times that pass's time.  Everywhere else it is
 * LA_PHI_FAVOR.  Both FAVOR+ forms evaluate the features of a query row
 * shifted by a constant of that row, and every key of a (batch, head) by one
 * constant taken from its first key; both constants cancel in the ratio,
 * keep the features' products inside fp32's range for large norms, and are
 * taken out of the returned S_N, z_N (and put into a given S0, z0). */
typedef enum la_phi_kind {
  LA_PHI_ELU1 = 0,
  LA_PHI_FAVOR = 1,
  LA_PHI_IDENTITY = 2,
  LA_PHI_FAVOR_PRECISE = 3
} la_phi_kind;

/* Number of kernels la_forward enqueues (per-span state, span scan, output). */
#define LA_FORWARD_KERNELS 3

/*
 * Workspace bytes la_forward needs for these arguments (fp32 per-span states:
 * B*H*(n_span+1)*(r*d_v + r)*4).  A head's chunks are split as evenly as
 * possible over n_span spans (one workgroup each); n_span is chosen by the
 * library from B*H, N, d, chunk and the I/O type so that the workgroups fill
 * the GPU in one round (the current device's compute units times the
 * workgroups per CU of the output kernel).  A span length set with
 * la_set_span_tokens replaces that choice; la_forward refuses a workspace
 * smaller than what its own call needs (LA_ERR_WORKSPACE), so a change in
 * between cannot go unnoticed.  Returns 0 for invalid or unsupported
 * arguments.
 */
size_t la_forward_workspace_bytes(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int causal,
                                  int chunk);

/*
 * Process-wide span length for the chunkwise prefill entry points, in tokens
 * (a multiple of 16; a value that is not a multiple of a call's chunk is
 * ignored by that call); 0 restores the library's own choice.  For tests and
 * tuning: it forces several spans per head (and with them the span scan) at
 * small N.  Thread-safe; affects calls made after it returns.
 * Errors: LA_ERR_SHAPE for a negative value, one above 2^24 or one that is
 * not a multiple of 16.
 */
la_status la_set_span_tokens(int tokens);
int la_get_span_tokens(void);

/*
 * How la_forward will run this shape (no device work): *n_span receives the
 * number of spans per head (workgroups per head); *single_pass receives 0,
 * since every shape runs the three-kernel path (span states, span scan,
 * outputs).  Either pointer may be NULL.  Errors as la_forward's shape
 * checks.
 */
la_status la_forward_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int causal, int chunk,
                            int *n_span, int *single_pass);

/*
 * Prefill: O = causal (or non-causal) linear attention of Q, K, V, evaluated
 * chunkwise ("Efficient attention variants" sec. 8: parallel inside a chunk,
 * state passed between chunks).  The result equals the token recurrence up to
 * rounding for every chunk size; chunk = 0 means 64.
 *
 *   Q, K, V  in:  device, io_dtype, layouts above.
 *   O        out: device, io_dtype [B][H][N][d_v]; may not alias Q, K or V.
 *   omega    in:  device fp32 [r][d] for LA_PHI_FAVOR, else ignored (may be NULL).
 *   S0, z0   in:  optional initial state (both NULL = zero state, "state reset");
 *                 if one is given the other must be too.
 *   S_out, z_out out: optional final state S_N, z_N (fp32), for handing the
 *                 prefix to la_decode_step or to a later la_forward call.
 *                 Non-causal: the full sums (including S0, z0).
 *   workspace    device scratch of at least la_forward_workspace_bytes(...);
 *                 contents on entry are ignored; owned by the caller.
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_UNSUPPORTED, LA_ERR_ALIGN,
 * LA_ERR_WORKSPACE (nothing enqueued), LA_ERR_HIP (launch failed).
 */
la_status la_forward(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d, int d_v,
                     int io_dtype, int phi, int r, const float *omega, int causal, int chunk, const float *S0,
                     const float *z0, float *S_out, float *z_out, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * la_forward plus timing: events is NULL or an array of 2*LA_FORWARD_KERNELS
 * hipEvent_t created by the caller (see la_event_create); events[2i] is
 * recorded on the stream before kernel i and events[2i+1] after it.
 * Kernels: 0 = per-span state, 1 = span scan, 2 = output.
 */
la_status la_forward_timed(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d,
                           int d_v, int io_dtype, int phi, int r, const float *omega, int causal, int chunk,
                           const float *S0, const float *z0, float *S_out, float *z_out, void *workspace,
                           size_t workspace_bytes, void *stream, void *const *events);

/*
 * la_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and errors as la_forward, except that the span states live in a
 * fixed scratch array of LA_NOALLOC_SCRATCH_BYTES bytes inside the library,
 * of which each GPU holds one copy from its first call until the process
 * ends (its device address is looked up once per device).  A call whose
 * workspace (la_forward_workspace_bytes) would exceed that size returns
 * LA_ERR_SCRATCH before any device call; use la_forward with a workspace for
 * such shapes.  The function calls no hipMalloc, hipFree or other
 * allocating routine.  Every call on one GPU shares that GPU's scratch, so
 * calls that overlap on one GPU (different streams, different threads
 * without ordering between them) race and give wrong results; calls
 * ordered on one stream are safe.  Nothing in the scratch has to start at
 * zero: every call writes each span state it reads.
 */
#define LA_NOALLOC_SCRATCH_BYTES (32u << 20)
la_status la_forward_noalloc(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d,
                             int d_v, int io_dtype, int phi, int r, const float *omega, int causal, int chunk,
                             const float *S0, const float *z0, float *S_out, float *z_out, void *stream);

/*
 * Decode step for B*H independent sequences/heads ("Efficient attention
 * variants" sec. 5; "Recurrent form" of the linear-attention-kernel page):
 *   S_new = S + phi(k) v^T, z_new = z + phi(k), o = phi(q)^T S_new / phi(q)^T z_new.
 *   S, z        in:  fp32 [B][H][r][d_v], [B][H][r].
 *   q, k, v     in:  io_dtype [B][H][d], [B][H][d], [B][H][d_v].
 *   o           out: io_dtype [B][H][d_v].
 *   S_new, z_new out: fp32; may alias S, z exactly (in-place update) but must
 *                not partially overlap them.
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_UNSUPPORTED, LA_ERR_ALIGN, LA_ERR_HIP.
 */
la_status la_decode_step(const float *S, const float *z, const void *q, const void *k, const void *v, void *o,
                         float *S_new, float *z_new, int B, int H, int d, int d_v, int io_dtype, int phi, int r,
                         const float *omega, void *stream);

/*
 * Causal prefill with a fixed per-head decay ("Efficient attention variants"
 * sec. 7.1, RetNet): S_t = gamma_h S_{t-1} + phi(k_t) v_t^T,
 * z_t = gamma_h z_{t-1} + phi(k_t), so that token j enters o_t with weight
 * gamma_h^(t-j) phi(q_t).phi(k_j); o_t = phi(q_t)^T S_t / phi(q_t)^T z_t, or
 * phi(q_t)^T S_t when normalize = 0.  gamma_h = 1 gives la_forward's causal
 * result.  An initial state S0, z0 is decayed like any earlier token: it
 * enters o_t (0-based) with gamma_h^(t+1).
 *   gamma     in: device fp32 [H], one decay per head (shared by the B
 *             sequences), each in (0, 1]; other values are not rejected
 *             (they are not read on the host) and give undefined results.
 *   normalize 1 (divide by phi(q)^T z) or 0.
 *   The other arguments are la_forward's with causal = 1 and no omega
 *   (FAVOR+ returns LA_ERR_UNSUPPORTED).  The workspace
 *   la_forward_workspace_bytes(..., causal = 1, chunk) returns is enough.
 * Errors: as la_forward; LA_ERR_NULL for a NULL gamma.
 */
la_status la_forward_decay(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d,
                           int d_v, int io_dtype, int phi, int r, const float *gamma, int normalize, int chunk,
                           const float *S0, const float *z0, float *S_out, float *z_out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Spans per head la_forward_decay uses for this shape (*n_span; may be NULL);
 * errors as its shape checks.  No device work. */
la_status la_forward_decay_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                                  int *n_span);

/* la_forward_decay plus timing events, as la_forward_timed. */
la_status la_forward_decay_timed(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d,
                                 int d_v, int io_dtype, int phi, int r, const float *gamma, int normalize, int chunk,
                                 const float *S0, const float *z0, float *S_out, float *z_out, void *workspace,
                                 size_t workspace_bytes, void *stream, void *const *events);

/*
 * Decode step with a fixed per-head decay (sec. 7.1):
 *   S_new = gamma_h S + phi(k) v^T, z_new = gamma_h z + phi(k),
 *   o = phi(q)^T S_new / phi(q)^T z_new (normalize = 1) or phi(q)^T S_new.
 * gamma: device fp32 [H] in (0, 1]; other arguments as la_decode_step
 * (ELU1/IDENTITY only).
 * Errors: as la_decode_step; LA_ERR_NULL for a NULL gamma.
 */
la_status la_decode_step_decay(const float *S, const float *z, const void *q, const void *k, const void *v,
                               void *o, float *S_new, float *z_new, int B, int H, int d, int d_v, int io_dtype,
                               int phi, int r, const float *gamma, int normalize, void *stream);

/*
 * Causal prefill with a per-token scalar gate ("Linear attention and SSM",
 * Mamba-2 SSD section, eq. of M = (C B^T) o L with A_t = a_t I):
 *   S_t = a_t S_{t-1} + phi(k_t) v_t^T,  z_t = a_t z_{t-1} + phi(k_t),
 * so that token j enters o_t with weight (a_{j+1} ... a_t) phi(q_t).phi(k_j);
 * o_t = phi(q_t)^T S_t / phi(q_t)^T z_t, or phi(q_t)^T S_t when
 * normalize = 0 (the page's structured masked attention with the feature
 * map applied to Q and K).  All gates one gives la_forward's causal result;
 * a constant gate per head gives la_forward_decay's.  An initial state S0,
 * z0 enters o_t (0-based) with a_0 ... a_t.
 *   log_a     in: device fp32 [B][H][N], the natural log of each gate
 *             (<= 0; Mamba-2 forms it as -Delta_t * A).  The kernels use
 *             max(log2 a_t, -126): a gate below 2^-126, zero (-inf) included,
 *             acts as 2^-126.  Positive values are not rejected (they are not
 *             read on the host) and give gates above one.  Inside a chunk
 *             the gate products are formed as 2^(c_i - c_j) from running
 *             fp32 sums c of log2 gates, so a weight's relative error grows
 *             with |c| (about |c| * 2^-23; with gates of Mamba-2's range
 *             |c| stays below a few hundred).
 *   normalize 1 (divide by phi(q)^T z) or 0.
 *   workspace at least la_forward_gated_workspace_bytes(...) bytes (the span
 *             states plus one fp32 total gate per (head, span)).
 *   The other arguments are la_forward's with causal = 1 and no omega
 *   (FAVOR+ returns LA_ERR_UNSUPPORTED).
 * Errors: as la_forward; LA_ERR_NULL for a NULL log_a.
 */
la_status la_forward_gated(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d,
                           int d_v, int io_dtype, int phi, int r, const float *log_a, int normalize, int chunk,
                           const float *S0, const float *z0, float *S_out, float *z_out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Workspace bytes la_forward_gated needs (0 for invalid or unsupported
 * arguments); the span length is chosen as for la_forward_workspace_bytes. */
size_t la_forward_gated_workspace_bytes(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r,
                                        int chunk);

/* Spans per head la_forward_gated uses for this shape (*n_span; may be NULL);
 * errors as its shape checks.  No device work. */
la_status la_forward_gated_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                                  int *n_span);

/* la_forward_gated plus timing events, as la_forward_timed. */
la_status la_forward_gated_timed(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d,
                                 int d_v, int io_dtype, int phi, int r, const float *log_a, int normalize, int chunk,
                                 const float *S0, const float *z0, float *S_out, float *z_out, void *workspace,
                                 size_t workspace_bytes, void *stream, void *const *events);

/*
 * Decode step with a per-token scalar gate:
 *   S_new = a S + phi(k) v^T, z_new = a z + phi(k),
 *   o = phi(q)^T S_new / phi(q)^T z_new (normalize = 1) or phi(q)^T S_new.
 * log_a: device fp32 [B][H], the natural log of this token's gate per
 * sequence and head (clamped as in la_forward_gated); other arguments as
 * la_decode_step (ELU1/IDENTITY only).
 * Errors: as la_decode_step; LA_ERR_NULL for a NULL log_a.
 */
la_status la_decode_step_gated(const float *S, const float *z, const void *q, const void *k, const void *v,
                               void *o, float *S_new, float *z_new, int B, int H, int d, int d_v, int io_dtype,
                               int phi, int r, const float *log_a, int normalize, void *stream);

/*
 * Causal prefill with a gate per token and key channel ("Efficient attention
 * variants" sec. 7.2, GLA; the RWKV-5/6 update of "Linear attention and SSM"
 * has the same shape):
 *   S_t = diag(a_t) S_{t-1} + phi(k_t) v_t^T,  z_t = a_t * z_{t-1} + phi(k_t),
 * so that token j enters o_t with weight sum_f phi(q_t)_f phi(k_j)_f
 * a_{j+1,f} ... a_{t,f}; o_t = phi(q_t)^T S_t / phi(q_t)^T z_t, or
 * phi(q_t)^T S_t when normalize = 0.  All gates one gives la_forward's causal
 * result; the same gate on every channel gives la_forward_gated's.  An
 * initial state S0, z0 enters o_t through channel f with a_{0,f} ... a_{t,f}.
 *   log_a     in: device fp32 [B][H][N][r], the natural log of each gate
 *             (<= 0; GLA forms a_t = sigmoid(x_t)^(1/16) per channel).  The
 *             kernels use max(log2 a, -14): a gate below 2^-14 (about 6.1e-5),
 *             zero included, acts as 2^-14, so that the factors the
 *             within-block weights are split into (16-token blocks, a
 *             reference at each half block) stay finite for features below
 *             2^16 in magnitude; GLA's gates stay far above the floor.
 *             Positive values are not rejected and give gates above one.
 *   normalize 1 (divide by phi(q)^T z) or 0.
 *   chunk     see the supported shapes; 0 means 64 (32 at d = 128).
 *   workspace at least la_forward_gla_workspace_bytes(...) bytes (the span
 *             states plus r fp32 total gates per (head, span)).
 *   The other arguments are la_forward's with causal = 1 and no omega.
 *   Also N must satisfy (N + 128) * r * 4 < 2^31 (LA_ERR_SHAPE otherwise).
 * Errors: as la_forward; LA_ERR_NULL for a NULL log_a.
 */
la_status la_forward_gla(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d,
                         int d_v, int io_dtype, int phi, int r, const float *log_a, int normalize, int chunk,
                         const float *S0, const float *z0, float *S_out, float *z_out, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Workspace bytes la_forward_gla needs (0 for invalid or unsupported
 * arguments); the span length is chosen as for la_forward_workspace_bytes. */
size_t la_forward_gla_workspace_bytes(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk);

/* Spans per head (*n_span) and chunk (*chunk_used) la_forward_gla uses for
 * this shape; either pointer may be NULL; errors as its shape checks.  No
 * device work. */
la_status la_forward_gla_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                                int *n_span, int *chunk_used);

/* la_forward_gla plus timing events, as la_forward_timed. */
la_status la_forward_gla_timed(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int d,
                               int d_v, int io_dtype, int phi, int r, const float *log_a, int normalize, int chunk,
                               const float *S0, const float *z0, float *S_out, float *z_out, void *workspace,
                               size_t workspace_bytes, void *stream, void *const *events);

/*
 * Decode step with a gate per key channel:
 *   S_new = diag(a) S + phi(k) v^T, z_new = a * z + phi(k),
 *   o = phi(q)^T S_new / phi(q)^T z_new (normalize = 1) or phi(q)^T S_new.
 * log_a: device fp32 [B][H][r], natural logs of this token's gates (clamped
 * as in la_forward_gla); other arguments as la_decode_step (ELU1/IDENTITY).
 * Errors: as la_decode_step; LA_ERR_NULL for a NULL log_a.
 */
la_status la_decode_step_gla(const float *S, const float *z, const void *q, const void *k, const void *v, void *o,
                             float *S_new, float *z_new, int B, int H, int d, int d_v, int io_dtype, int phi, int r,
                             const float *log_a, int normalize, void *stream);

/* Number of kernels la_backward enqueues (forward span states, their scan,
 * the dQ pass, the reverse scan, the dK/dV pass). */
#define LA_BACKWARD_KERNELS 5

/*
 * Backward pass of the causal normalised output (no initial state): for an
 * upstream gradient dO, the gradients of sum(dO * O) with respect to Q, K
 * and V.  The pages define the forward ("Efficient attention variants"
 * sec. 5) and name the backward among the costs that decide speed (sec. 8)
 * without deriving it; what is computed is the chain rule on that forward:
 * with D_i = phi(q_i).z_i, g_i = dO_i / D_i, h_i = -(dO_i . O_i) / D_i,
 *   dphi(q_i) = sum_{j<=i} (v_j.g_i + h_i) phi(k_j),
 *   dphi(k_j) = sum_{i>=j} (v_j.g_i + h_i) phi(q_i),
 *   dv_j      = sum_{i>=j} (phi(q_i).phi(k_j)) g_i,
 * and dq = dphi(q) * phi'(q), dk = dphi(k) * phi'(k) (phi' of ELU+1 with
 * alpha = 1: 1 for x > 0, e^x otherwise; 1 for the identity).  Evaluated
 * chunkwise: a forward-direction pass for dQ (with the forward's span
 * prefix states) and a reverse-direction pass for dK, dV (with suffix states
 * of phi(q) g^T and phi(q) h), bf16 operands and fp32 accumulation.
 *   Q, K, V, O, dO in:  device bf16, O the forward output of la_forward
 *                  (causal, same phi) for these Q, K, V; layouts as la_forward.
 *   dQ, dK, dV     out: device bf16, the shapes of Q, K, V; may not alias the
 *                  inputs.
 *   workspace      device scratch of at least la_backward_workspace_bytes(...).
 * Supported: bf16, ELU1/IDENTITY, d = d_v in {64, 128}, chunk 64 (0 means 64);
 * others return LA_ERR_UNSUPPORTED.
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_UNSUPPORTED, LA_ERR_ALIGN,
 * LA_ERR_WORKSPACE (nothing enqueued), LA_ERR_HIP.
 */
la_status la_backward(const void *Q, const void *K, const void *V, const void *O, const void *dO, void *dQ, void *dK,
                      void *dV, int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes la_backward needs (0 for invalid or unsupported arguments):
 * two sets of fp32 span states and (D_i, h_i) per token. */
size_t la_backward_workspace_bytes(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk);

/* Spans per head la_backward uses (*n_span; may be NULL); no device work. */
la_status la_backward_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                             int *n_span);

/* la_backward plus timing: events NULL or 2*LA_BACKWARD_KERNELS hipEvent_t,
 * events[2i] recorded before kernel i and events[2i+1] after it. */
la_status la_backward_timed(const void *Q, const void *K, const void *V, const void *O, const void *dO, void *dQ,
                            void *dK, void *dV, int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r,
                            int chunk, void *workspace, size_t workspace_bytes, void *stream, void *const *events);

/*
 * Standalone feature map: Y[i] = phi(X[i]) for rows i = 0..rows-1.
 *   X in: io_dtype [rows][d];  Y out: fp32 [rows][r];  omega as in la_forward.
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_UNSUPPORTED, LA_ERR_ALIGN, LA_ERR_HIP.
 */
la_status la_feature_map(const void *X, float *Y, long long rows, int d, int io_dtype, int phi, int r,
                         const float *omega, void *stream);

/* Static, human-readable text for a status code. */
const char *la_status_string(int status);

/* Text of the HIP runtime error behind the most recent LA_ERR_HIP returned
 * to the calling thread ("" if none).  Static storage; do not free. */
const char *la_hip_error_string(void);

/* Library ABI version (major * 100 + minor). */
int la_version(void);

/* Event helpers for la_forward_timed (thin wrappers over hipEvent*).  The
 * events are for timing only: they are created with
 * hipEventDisableSystemFence, so recording one performs no system-scope
 * fence (cache write-back and invalidate) and does not slow the kernels that
 * follow.  Read elapsed times after synchronising the device (or the
 * stream); the events do not order host-visible memory. */
la_status la_event_create(void **event);
la_status la_event_destroy(void *event);
la_status la_event_elapsed_ms(void *start, void *end, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_LA_H */
