/*
 * linattn.h -- C ABI of the MI355X (gfx950) causal linear-attention library.
 *
 * Eight operations, each a hand-written HIP path:
 *   la_forward               chunked prefill of causal ELU+1 linear attention
 *   delta_forward            chunked prefill of the delta-rule fast-weight memory
 *   gated_delta_forward      the same with a per-token forgetting gate
 *   ssd_forward              chunked prefill of the scalar-decay memory (Mamba-2 / SSD form)
 *   la_decode_step           one-token decode of ELU+1 linear attention on a resident state
 *   delta_decode_step        one-token decode of the delta rule on a resident state
 *   gated_delta_decode_step  the same with a forgetting gate
 *   ssd_decode_step          one-token decode of the scalar-decay memory
 *   la_backward              gradients of la_forward (training, with recomputation)
 *   delta_backward           gradients of delta_forward / gated_delta_forward
 * a training pair for the delta rule that keeps the forward's context for
 * the backward instead of recomputing it: delta_forward_train,
 * delta_backward_after_forward;
 * two delta-rule calls with serving options (input transforms, the
 * read-then-write prediction as an extra output): delta_forward_ex,
 * delta_decode_step_ex; and the prefills over packed batches of
 * variable-length sequences, each sequence starting from its own state:
 * la_forward_packed, delta_forward_packed, ssd_forward_packed.
 *
 * Pages the definitions come from:
 *   [LinearMem]  "AIGC 基本功｜线性、循环与记忆架构-LinearMem"
 *   [Recurrence] "手撕：递推与记忆模型"
 *   [LA-SSM]     "线性注意力与 SSM:两条技术路线的完整推导"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are contiguous, row-major, in DEVICE memory of the current HIP
 *   device.  q, k, v, beta and o have the element type `dtype` (LA_F32 =
 *   IEEE fp32, LA_BF16 = bfloat16 bits); states S and z are always fp32.
 * - Shapes: q, k [B][H][T][dk]; v, o [B][H][T][dv]; beta [B][H][T];
 *   S [B][H][dk][dv] (key-first: S = sum phi(k) v^T, read as phi(q)^T S,
 *   [LinearMem] §03); z [B][H][dk].  Decode uses N in place of B and no T.
 * - Ownership: the caller owns every buffer, including the workspace.  The
 *   library allocates no device memory; its only state between calls is a
 *   process-wide counter that tags la_forward's look-back flags.  No result
 *   carries over from one call to the next unless passed in as an initial
 *   state ([LinearMem] §05: reset per request by zeroing a slot), with one
 *   exception: delta_backward_after_forward reads the context that
 *   delta_forward_train left in the workspace passed to both.  One
 *   workspace must not serve two calls that may run at the same time.
 * - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *   stream) and the call returns without synchronising.  Execution-time
 *   faults surface at the caller's next synchronisation.
 * - Validation first: arguments are checked before anything is launched; on
 *   any non-OK status nothing has been enqueued and no buffer was written.
 *   la_last_error() then describes the problem (per calling thread).
 * - Supported: dk, dv in {64, 128}; chunk == 64, and for la_forward and
 *   delta_forward on uniform batches also 16, 32 and 128 (la_forward with
 *   LA_F32: 16 and 32); dtype LA_BF16
 *   everywhere and LA_F32 for la_forward (at chunk 64, dk = 128 with
 *   dv = 128 excluded) and the decode steps.  Forgetting gates alpha are
 *   fp32 for every dtype.
 *   Other valid-but-unsupported sizes return LA_ERR_UNSUPPORTED.
 * - Non-finite inputs are not checked and propagate.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/*
 * Input transforms of the delta-rule *_ex calls (bit flags).  [LinearMem]
 * §05: FLA hands the q/k L2 normalisation and the gate and beta transforms
 * to the kernel; §08: production models predict a raw gate that a
 * non-linearity in the kernel turns into the step size.
 *   LA_NORMALIZE_QK  each q_t and k_t is scaled to unit L2 norm before use
 *                    (a zero vector stays zero);
 *   LA_BETA_SIGMOID  beta holds logits; the rule uses sigmoid(beta).
 */
enum { LA_NORMALIZE_QK = 1, LA_BETA_SIGMOID = 2 };

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, eps <= 0, bad dtype or chunk */
    LA_ERR_UNSUPPORTED = 2, /* a valid configuration the library has no kernel for         */
    LA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the *_workspace_bytes query   */
    LA_ERR_HIP = 4          /* a HIP launch failed; la_last_error() has the HIP message      */
} la_status;

/*
 * Bytes of device workspace la_forward needs for these sizes; 0 if the
 * sizes are invalid.  The workspace holds 64-bit look-back flags, two fp32
 * (S, z) per head and segment of the sequence, and room for one copy of the
 * initial state (taken when S_out, z_out alias S0, z0).  Its contents need no
 * initialisation: each flag carries the tag of the call that wrote it, and a
 * call recorded into a HIP graph (replayed with one tag) clears the flags in
 * a launch of its own first.
 */
size_t la_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);

/*
 * Causal ELU+1 linear attention over a whole sequence (prefill).
 * [LinearMem] §03: phi(u) = u + 1 (u > 0), exp(u) (u <= 0);
 *   S_t = S_{t-1} + phi(k_t) v_t^T,  z_t = z_{t-1} + phi(k_t),
 *   o_t^T = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps)     (write, then read).
 * S0, z0   initial state; NULL means zero (the page's S_0 = 0, z_0 = 0).
 * o        [B][H][T][dv] output, dtype.
 * S_out, z_out  final state S_T, z_T (fp32); NULL means not returned.  They
 *          may alias S0, z0 (continue a sequence in place, the initial/final
 *          state hand-off of [Recurrence] "Chunked scan").
 * eps      > 0; the pages use 1e-6.
 * chunk    tokens per chunk: 64 (one fused launch), or 16, 32, 128 (LA_F32:
 *          16, 32), a blocked path of three launches (segment sums, their
 *          prefix, chunk loops of `chunk` tokens).  The result does not
 *          depend on it beyond rounding ([Recurrence] "Chunked scan": a scan
 *          handed its state every few tokens equals one pass; [LA-SSM] §3,
 *          the chunkwise form); the workspace size does
 *          (la_forward_workspace_bytes with the same chunk).
 * Errors: LA_ERR_INVALID_ARG (q, k, v or o NULL; B, H, T, dk, dv < 1; eps not
 * > 0 or not finite; chunk < 1; dtype unknown), LA_ERR_UNSUPPORTED (other
 * chunk sizes, dims), LA_ERR_WORKSPACE, LA_ERR_HIP.
 */
la_status la_forward(const void* q, const void* k, const void* v,
                     const float* S0, const float* z0,
                     void* o, float* S_out, float* z_out,
                     int B, int H, int T, int dk, int dv, int dtype, float eps, int chunk,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * TEST HOOK: la_forward with the look-back's wait bound chosen by the caller.
 * la_forward cuts each sequence into segments, one workgroup each; a
 * workgroup finds the state entering its segment by polling its
 * predecessors' published sums ([Recurrence] "Chunked scan": only the state
 * crosses a boundary), at most `lookback_polls` times per window of
 * predecessors (la_forward uses 4000), and otherwise recomputes that state
 * from the inputs with the same additions in the same order, so the result
 * is the same bit for bit.  lookback_polls < 0 skips the polling: every
 * segment but the first of its sequence recomputes.  Meant for tests of that
 * path; the recomputation costs O(segments^2) per sequence.  Arguments,
 * workspace and errors are those of la_forward.
 */
la_status la_forward_lookback_polls(const void* q, const void* k, const void* v,
                                    const float* S0, const float* z0,
                                    void* o, float* S_out, float* z_out,
                                    int B, int H, int T, int dk, int dv, int dtype, float eps, int chunk,
                                    void* workspace, size_t workspace_bytes, void* stream, int lookback_polls);

/*
 * la_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  The workspace is a fixed scratch array in device
 * memory, LA_NOALLOC_SCRATCH_BYTES per GPU the library runs on, held until
 * the process ends; the call itself allocates and frees nothing.
 * Arguments, results and errors are those of la_forward, plus
 * LA_ERR_UNSUPPORTED when these sizes need more workspace than the scratch
 * holds (la_forward_workspace_bytes(...) > LA_NOALLOC_SCRATCH_BYTES; the
 * long-stream size B=1, H=32, T=65536, dk=dv=64 fits).
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (other streams, other host threads) race and must not be issued.
 * What a call leaves in the scratch never changes a later call's result.
 */
#define LA_NOALLOC_SCRATCH_BYTES (96u << 20)
la_status la_forward_noalloc(const void* q, const void* k, const void* v,
                             const float* S0, const float* z0,
                             void* o, float* S_out, float* z_out,
                             int B, int H, int T, int dk, int dv, int dtype, float eps, int chunk,
                             void* stream);

/*
 * Bytes of device workspace delta_forward (and gated_delta_forward,
 * delta_forward_ex) needs; 0 if the sizes are invalid.  The workspace holds
 * the per-segment affine maps and states (fp32) and, at chunk 64, one record
 * per chunk of the chunk's triangular inverse T = (I + A)^{-1} (bf16, 8 KiB).
 */
size_t delta_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);

/*
 * Delta-rule fast-weight memory over a whole sequence (prefill).
 * [LinearMem] §03 "从累加改成纠错" and [Recurrence] "Delta-rule fast weight":
 *   S_t = S_{t-1} + beta_t k_t (v_t^T - k_t^T S_{t-1})
 * with no feature map and no normaliser.  The output is the write-then-read
 * query read o_t = S_t^T q_t (raw q).  Keys are used as given: the exact
 * overwrite property needs unit keys, which the caller provides.
 * beta     [B][H][T], dtype: the final per-token step size (no transform).
 * S0       initial state, NULL = zero.  S_out final state (may alias S0), or NULL.
 * chunk    64, or 16, 32, 128: a blocked path (segment maps by chunk loops of
 *          `chunk` tokens, their composition, chunk loops writing o) whose
 *          result matches the 64-token one up to rounding ([Recurrence]
 *          "Chunked scan").  gated_delta_forward, delta_forward_ex and the
 *          packed batches take 64 only (others: LA_ERR_UNSUPPORTED).
 * Errors: as la_forward (beta NULL is LA_ERR_INVALID_ARG).
 */
la_status delta_forward(const void* q, const void* k, const void* v, const void* beta,
                        const float* S0, void* o, float* S_out,
                        int B, int H, int T, int dk, int dv, int dtype, int chunk,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of ELU+1 linear attention on a resident fp32 state,
 * updated IN PLACE ([LinearMem] §03 recurrence; §05 in-place inference update):
 *   S <- S + phi(k) v^T,  z <- z + phi(k),  o = phi(q)^T S / (phi(q)^T z + eps).
 * q, k [N][H][dk]; v, o [N][H][dv] (dtype); S [N][H][dk][dv], z [N][H][dk] fp32.
 * Errors: LA_ERR_INVALID_ARG (a pointer NULL, N, H, dk, dv < 1, eps not > 0,
 * dtype unknown), LA_ERR_UNSUPPORTED, LA_ERR_HIP.
 */
la_status la_decode_step(const void* q, const void* k, const void* v,
                         float* S, float* z, void* o,
                         int N, int H, int dk, int dv, int dtype, float eps, void* stream);

/* Static text for a status code. */
const char* la_status_string(int status);

/* Detail for the last non-OK status returned on the calling thread ("" if none). */
const char* la_last_error(void);

/*
 * One decode step of the delta-rule fast-weight memory on a resident fp32
 * state, updated IN PLACE ([LinearMem] §03 "从累加改成纠错", [Recurrence]
 * "Delta-rule fast weight"; [LinearMem] §05 in-place inference update):
 *   u = v - S^T k,  S <- S + beta k u^T,  o = S^T q   (write, then read),
 * the single-token form of delta_forward (no feature map, no normaliser;
 * keys used as given).
 * q, k [N][H][dk]; v, o [N][H][dv]; beta [N][H] (dtype); S [N][H][dk][dv] fp32.
 * Errors: LA_ERR_INVALID_ARG (a pointer NULL, N, H, dk, dv < 1, dtype
 * unknown, S not 16-byte aligned), LA_ERR_UNSUPPORTED (dk or dv not in
 * {64, 128}), LA_ERR_HIP.
 */
la_status delta_decode_step(const void* q, const void* k, const void* v, const void* beta, float* S,
                            void* o, int N, int H, int dk, int dv, int dtype, void* stream);

/*
 * delta_forward / gated_delta_forward with serving options: alpha NULL is the
 * plain delta rule, non-NULL the gated rule (fp32 [B][H][T]); `flags` selects
 * the input transforms above; `pred` (optional, [B][H][T][dv], dtype)
 * receives the prediction made before each write,
 *   pred_t = (alpha_t S_{t-1})^T k_t = v_t - u_t,
 * the read-then-write sequence of [Recurrence] "Delta-rule fast weight"
 * (whose reference loop returns these reads).  Errors: as delta_forward, plus
 * LA_ERR_INVALID_ARG for unknown flags or a misaligned pred.
 */
la_status delta_forward_ex(const void* q, const void* k, const void* v, const void* beta,
                           const float* alpha, const float* S0, void* o, float* S_out,
                           void* pred, int flags,
                           int B, int H, int T, int dk, int dv, int dtype, int chunk,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * delta_decode_step / gated_delta_decode_step with the same options: alpha
 * NULL = plain rule, else fp32 [N][H]; flags as above; pred (optional,
 * [N][H][dv], dtype) = (alpha S)^T k, the prediction before the write.
 */
la_status delta_decode_step_ex(const void* q, const void* k, const void* v, const void* beta,
                               const float* alpha, float* S, void* o, void* pred, int flags,
                               int N, int H, int dk, int dv, int dtype, void* stream);

/*
 * The gated delta rule over a whole sequence (prefill).  [LinearMem] §03:
 * the old state is first decayed by a forgetting factor, then corrected
 * against the decayed state (the order matters; this is the Gated DeltaNet
 * rule):
 *   S~ = alpha_t S_{t-1},  S_t = S~ + beta_t k_t (v_t^T - k_t^T S~),  o_t = S_t^T q_t.
 * alpha    [B][H][T] fp32 (whatever dtype is), each in (0, 1]; alpha = 1 is
 *          delta_forward.  A factor below e^-20 acts as e^-20 (a decay far
 *          below fp32 resolution, so alpha = 0 is an effective reset).
 * Other arguments, the workspace (size from delta_forward_workspace_bytes)
 * and the errors are those of delta_forward; alpha NULL is
 * LA_ERR_INVALID_ARG.
 */
la_status gated_delta_forward(const void* q, const void* k, const void* v, const void* beta,
                              const float* alpha, const float* S0, void* o, float* S_out,
                              int B, int H, int T, int dk, int dv, int dtype, int chunk,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of the gated delta rule on a resident fp32 state, updated
 * IN PLACE ([LinearMem] §03; §05 in-place inference update):
 *   S~ = alpha S,  u = v - S~^T k,  S <- S~ + beta k u^T,  o = S^T q.
 * alpha    [N][H] fp32 (whatever dtype is); alpha = 0 resets exactly.
 * Other arguments and the errors are those of delta_decode_step; alpha NULL
 * is LA_ERR_INVALID_ARG.
 */
la_status gated_delta_decode_step(const void* q, const void* k, const void* v, const void* beta,
                                  const float* alpha, float* S, void* o,
                                  int N, int H, int dk, int dv, int dtype, void* stream);

/* Bytes of device workspace ssd_forward needs; 0 if the sizes are invalid. */
size_t ssd_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);

/*
 * Scalar-decay linear memory over a whole sequence (prefill): the Mamba-2 /
 * SSD form of [LA-SSM] §3 (the outer-product state of linear attention with
 * a scalar decay on the old state), written key-first:
 *   S_t = alpha_t S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t   (write, then read),
 * no feature map, no normaliser.  With dk = dv = 1 it is the selective scan
 * of [Recurrence] "Selective scan" (a = alpha, b = k, x = v, c = q).
 * alpha    [B][H][T] fp32 (whatever dtype is), each in (0, 1]; a factor
 *          below e^-20 acts as e^-20 (an effective reset).
 * S0       initial state, NULL = zero; 16-byte aligned.  S_out final state
 *          (may alias S0), or NULL.
 * Supported: dtype LA_BF16; dk, dv in {64, 128}; chunk 64.
 * Errors: LA_ERR_INVALID_ARG (q, k, v, alpha or o NULL; sizes < 1; chunk < 1;
 * dtype unknown; misaligned pointers), LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE,
 * LA_ERR_HIP.
 */
la_status ssd_forward(const void* q, const void* k, const void* v, const float* alpha,
                      const float* S0, void* o, float* S_out,
                      int B, int H, int T, int dk, int dv, int dtype, int chunk,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of the scalar-decay memory on a resident fp32 state,
 * updated IN PLACE ([LA-SSM] §3; [LinearMem] §05 in-place inference update):
 *   S <- alpha S + k v^T,   o = S^T q.
 * q, k [N][H][dk]; v, o [N][H][dv] (dtype); alpha [N][H] fp32 (alpha = 0
 * resets exactly); S [N][H][dk][dv] fp32, 16-byte aligned.
 * Errors: LA_ERR_INVALID_ARG (a pointer NULL, sizes < 1, dtype unknown, S
 * misaligned), LA_ERR_UNSUPPORTED (dk or dv not in {64, 128}), LA_ERR_HIP.
 */
la_status ssd_decode_step(const void* q, const void* k, const void* v, const float* alpha, float* S,
                          void* o, int N, int H, int dk, int dv, int dtype, void* stream);

/*
 * Backward pass of la_forward (training).  [LinearMem] §03: storing every
 * step's state makes training memory grow with the length; chunking and
 * recomputation in the backward pass remove that cost (§06: training and
 * decoding are validated separately).  For the loss
 *   L = sum_t dO_t . o_t + <dS_T, S_T> + <dz_T, z_T>
 * this writes dq, dk [B][H][T][dk] and dv [B][H][T][dv] (dtype) and, if
 * non-NULL, dS0 [B][H][dk][dv], dz0 [B][H][dk] (fp32).  q, k, v, S0, z0, eps
 * as given to la_forward (its states are recomputed, nothing of the forward
 * call is needed); dO [B][H][T][dv] (dtype); dS_T, dz_T fp32 or NULL (zero).
 * Supported: dtype LA_BF16, dk, dv in {64, 128}, chunk 64.  Errors as
 * la_forward; workspace size from la_backward_workspace_bytes.
 */
size_t la_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);
la_status la_backward(const void* q, const void* k, const void* v, const float* S0, const float* z0,
                      const void* dO, const float* dS_T, const float* dz_T,
                      void* dq, void* dk_out, void* dv_out, float* dS0, float* dz0,
                      int B, int H, int T, int dk, int dv, int dtype, float eps, int chunk,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gradients of delta_forward (alpha NULL) or gated_delta_forward (alpha
 * given) for the linear loss L = sum_t dO_t . o_t + <dS_T, S_T>:
 * [LinearMem] §03 (the corrective write, its decayed variant, and training
 * by chunks with only chunk-boundary states kept and the rest recomputed).
 * Inputs as in the forward call (q, k, v, beta bf16; alpha fp32 [B][H][T] or
 * NULL; S0 fp32 or NULL = zero); dO bf16 [B][H][T][dv]; dS_T fp32
 * [B][H][dk][dv] or NULL = zero.  Outputs: dq, dk_out [B][H][T][dk] and
 * dv_out [B][H][T][dv] (bf16); dbeta fp32 [B][H][T]; dalpha fp32 [B][H][T],
 * required exactly when alpha is given (the forward clamps log alpha_t at
 * -20, so a gate below e^-20 gets gradient 0); dS0 fp32 [B][H][dk][dv] or
 * NULL.  Every output is overwritten.  bf16 only; uniform batches only.
 * The workspace (delta_backward_workspace_bytes) holds the forward's
 * workspace plus every chunk's entering state and leaving state gradient
 * (bf16), 4 * B * H * ceil(T / 64) * dk * dv bytes of it.
 */
size_t delta_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);
la_status delta_backward(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                         const float* S0, const void* dO, const float* dS_T,
                         void* dq, void* dk_out, void* dv_out, float* dbeta, float* dalpha, float* dS0,
                         int B, int H, int T, int dk, int dv, int dtype, int chunk,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training pair of the delta rule ([LinearMem] §03: in training by chunks,
 * the states at chunk boundaries are what the backward pass needs; keeping
 * them from the forward pass spares their recomputation).
 *
 * delta_forward_train: delta_forward (alpha NULL) or gated_delta_forward
 * (alpha given), with the same arguments, outputs and errors, bf16 only,
 * whose workspace is a delta_backward workspace (size from
 * delta_backward_workspace_bytes, 16-byte aligned; LA_ERR_WORKSPACE if
 * smaller).  Besides o and S_out it leaves in the workspace the context the
 * backward pass reads: every chunk's correction record, every segment's
 * affine map and entering state, and every 64-token chunk's entering state
 * as bf16 tiles.  o and S_out equal delta_forward's bit for bit.
 *
 * delta_backward_after_forward: delta_backward with the same arguments,
 * outputs and errors, given the workspace that a delta_forward_train call
 * on the same q, k, v, beta, alpha, S0 and sizes filled, unchanged since.
 * It skips the backward's forward sweep and returns delta_backward's results
 * bit for bit.  With any other workspace contents the results are
 * meaningless (nothing detects this); the workspace is overwritten, so a
 * second backward needs a second forward.
 */
la_status delta_forward_train(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                              const float* S0, void* o, float* S_out, int B, int H, int T, int dk, int dv,
                              int dtype, int chunk, void* workspace, size_t workspace_bytes, void* stream);
la_status delta_backward_after_forward(const void* q, const void* k, const void* v, const void* beta,
                                       const float* alpha, const float* S0, const void* dO, const float* dS_T,
                                       void* dq, void* dk_out, void* dv_out, float* dbeta, float* dalpha,
                                       float* dS0, int B, int H, int T, int dk, int dv, int dtype, int chunk,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed batches ([LinearMem] §05: when a request ends only its own state is
 * cleared, and samples concatenated without a reset would read one another;
 * [Recurrence] "验证边界": state resets at request, batch and document
 * boundaries).  N sequences of different lengths are concatenated along the
 * token axis: q, k [H][T_total][dk]; v, o, pred [H][T_total][dv]; beta,
 * alpha [H][T_total]; sequence n is rows cu[n] .. cu[n+1]-1 of every head.
 * Each sequence starts from its own initial state (S0, z0 [N][H][..], NULL =
 * zero) and returns its own final state (S_out, z_out [N][H][..]); no
 * information crosses a sequence boundary.  Results equal the per-sequence
 * calls.
 * cu_seqlens       device int32 [N+1]: 0 = cu[0] < cu[1] < ... < cu[N] = T_total
 *                  (no empty sequence); the kernels read it.
 * cu_seqlens_host  host int32 [N+1], the same values; the call plans its
 *                  launches from it and validates it (LA_ERR_INVALID_ARG).
 *                  Device offsets that differ from it give wrong results but
 *                  never an access outside the inputs, outputs or workspace.
 * The workspace (size from the matching *_packed_workspace_bytes query, which
 * needs only the host offsets) also holds a per-sequence segment table the
 * call builds on the device.  Other arguments and errors are those of the
 * uniform calls.
 */
size_t la_forward_packed_workspace_bytes(const int* cu_seqlens_host, int N, int H, int T_total,
                                         int dk, int dv, int chunk);
la_status la_forward_packed(const void* q, const void* k, const void* v,
                            const int* cu_seqlens, const int* cu_seqlens_host, int N,
                            const float* S0, const float* z0, void* o, float* S_out, float* z_out,
                            int H, int T_total, int dk, int dv, int dtype, float eps, int chunk,
                            void* workspace, size_t workspace_bytes, void* stream);

size_t delta_forward_packed_workspace_bytes(const int* cu_seqlens_host, int N, int H, int T_total,
                                            int dk, int dv, int chunk);
/* The delta rule (alpha NULL) or the gated rule, with the options of delta_forward_ex. */
la_status delta_forward_packed(const void* q, const void* k, const void* v, const void* beta,
                               const float* alpha, const int* cu_seqlens, const int* cu_seqlens_host,
                               int N, const float* S0, void* o, float* S_out, void* pred, int flags,
                               int H, int T_total, int dk, int dv, int dtype, int chunk,
                               void* workspace, size_t workspace_bytes, void* stream);

size_t ssd_forward_packed_workspace_bytes(const int* cu_seqlens_host, int N, int H, int T_total,
                                          int dk, int dv, int chunk);
la_status ssd_forward_packed(const void* q, const void* k, const void* v, const float* alpha,
                             const int* cu_seqlens, const int* cu_seqlens_host, int N,
                             const float* S0, void* o, float* S_out,
                             int H, int T_total, int dk, int dv, int dtype, int chunk,
                             void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
