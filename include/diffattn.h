/*
 * diffattn.h -- C ABI of the MI355X (gfx950) differential-attention library.
 *
 * The library computes multi-head differential attention and its gradients:
 *
 *   O = (softmax(Q1 K1^T / sqrt(D) + M) - lambda * softmax(Q2 K2^T / sqrt(D) + M)) V
 *
 * as defined on the paperleet page "Differential Transformer Attention"
 * (equation for A1, A2 and O; M is 0 on allowed keys and -inf on future keys
 * under the causal mask, in both branches; softmax runs over keys), with
 * Q1, Q2, K1, K2 of shape [B, H, T, D] and V, O of shape [B, H, T, 2D].
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (HIP device memory) owned by the
 *     caller.  The library allocates nothing and keeps no state; every entry
 *     point is thread-safe.  (One exception: diffattn_decode_noalloc works in
 *     a device array the library holds per GPU; see there.)
 *   - Tensors are dense, contiguous and row-major in the shapes given.  Every
 *     tensor pointer must be 16-byte aligned.
 *   - Inputs are never written.  Outputs must not overlap any input.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising.  Argument checks run on the
 *     host before any HIP call, so an invalid call launches nothing.
 *   - Element type `dtype`: DIFFATTN_F32 (float) or DIFFATTN_BF16 (bfloat16).
 *     The output has the input dtype.  Accumulation is fp32 in both cases; in
 *     bf16 mode the probabilities are rounded to bf16 before they multiply V.
 *   - Head width D must be 32, 64 or 128 (V and O rows are 2D wide).
 *   - lambda is a per-head fp32 device array [H]; a per-layer scalar is the
 *     case of all heads equal.  It is not clamped: negative values and values
 *     above 1 are allowed (paperleet page, "Return requirements").
 *   - Size limits ("grid size" below; beyond them ERR_UNSUPPORTED, nothing
 *     launched).  Offsets between heads and batches are 64-bit, so tensors
 *     may exceed 4 GiB; within one (b, h) slice, T x (row width) must stay
 *     below 2^31 elements, and B x H below 2^31.  A dispatch holds at most
 *     2^32 - 1 work-items: prefill, training forward and backward need
 *     4 B H (T + 255) <= 2^32 - 1 (every one of their launches runs at most 4
 *     work-items per row of its padded row range; this only binds beyond
 *     2^30 rows, far past one GPU's memory); decode needs B H S <= 2^24 - 1
 *     split-K workgroups of 256 threads (S the split count; V2: B Hkv S);
 *     diffattn_lambda needs H <= 2^26 - 1 (one 64-thread workgroup per head).
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIFFATTN_OK = 0,
  DIFFATTN_ERR_INVALID = 1,     /* null pointer, size < 1, eps <= 0 with head norm,
                                   overlapping output, bad split count */
  DIFFATTN_ERR_UNSUPPORTED = 2, /* unknown dtype, D not in {32,64,128}, misaligned pointer,
                                   sizes beyond the 32-bit grid limits */
  DIFFATTN_ERR_WORKSPACE = 3,   /* decode/backward workspace or training saved-state
                                   buffer missing or too small */
  DIFFATTN_ERR_HIP = 4          /* the kernel launch itself failed */
} diffattn_status;

typedef enum { DIFFATTN_F32 = 0, DIFFATTN_BF16 = 1 } diffattn_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* diffattn_status_string(int status);

/*
 * lambda_init(l) = 0.8 - 0.6 * exp(-0.3 * (l - 1)) for layer l = 1, 2, ...
 * (aifetchly "Differential Transformer: Canceling LLM Attention Noise",
 * section 3; paperleet page, "Formula and conventions").  Host-only; returns
 * NaN for layer < 1.
 */
float diffattn_lambda_init(int layer);

/*
 * lambda_out[h] = exp(lq1[h] . lk1[h]) - exp(lq2[h] . lk2[h]) + lambda_init
 * (aifetchly page, section 3; paperleet page, scalar parameterisation).
 *
 *   lq1, lk1, lq2, lk2  device fp32 [H, Dl], row h = the four vectors of head h
 *   lambda_out          device fp32 [H]; may be passed straight to diffattn_fwd
 *                       or diffattn_decode on the same stream
 * Errors: ERR_INVALID for a null pointer, H < 1 or Dl < 1, or lambda_out
 * overlapping an input; ERR_UNSUPPORTED for a misaligned pointer (4 bytes
 * suffices here) or H beyond the grid limit.
 */
diffattn_status diffattn_lambda(const float* lq1, const float* lk1, const float* lq2,
                                const float* lk2, int H, int Dl, float lambda_init,
                                float* lambda_out, hipStream_t stream);

/*
 * Prefill forward (paperleet page, equation for A1, A2, O).
 *
 *   q1, k1, q2, k2  [B, H, T, D]   dtype elements
 *   v               [B, H, T, 2D]  dtype elements
 *   lambda          [H] fp32 (device)
 *   causal          non-zero: key j is visible to query i iff j <= i (top-left
 *                   aligned, both maps); zero: every key is visible
 *   headnorm        non-zero: each output row is divided by
 *                   sqrt(mean over its 2D channels of o^2 + eps) and multiplied
 *                   by (1 - lambda_init) (aifetchly page, section 4: per-head
 *                   normalisation then the (1 - lambda_init) multiplier; RMS
 *                   form, no affine weight).  zero: raw (A1 - lambda A2) V,
 *                   lambda_init and eps unused.
 *   out             [B, H, T, 2D]  dtype elements
 * Errors: ERR_INVALID (null pointer, B/H/T < 1, headnorm with eps <= 0 or NaN,
 * out overlapping an input), ERR_UNSUPPORTED (dtype, D, alignment, grid size),
 * ERR_HIP (launch failure).
 */
diffattn_status diffattn_fwd(int dtype, int B, int H, int T, int D, const void* q1,
                             const void* k1, const void* q2, const void* k2, const void* v,
                             const float* lambda, int causal, int headnorm, float lambda_init,
                             float eps, void* out, hipStream_t stream);

/*
 * Prefill on strided views, read and written in place (no copies): the
 * aifetchly page ("Differential Transformer: Canceling LLM Attention Noise",
 * its numpy forward, step 1) cuts Q1, Q2 (and K1, K2) out of one projection
 * of width 2D along the feature axis, and the paperleet page's interface
 * section allows strided inputs.  Q1 = Q[..., :D] and Q2 = Q[..., D:] of a
 * fused [B, T, H, 2D] projection, for instance, are views with row stride
 * 2HD, head stride 2D and batch stride 2THD elements.
 *
 *   strides  HOST array of 18 int64: for q1, k1, q2, k2, v, out in turn the
 *            batch, head and row stride in elements (the tensors keep their
 *            logical [B, H, T, D] / [B, H, T, 2D] shapes; the last dimension
 *            is contiguous).  Every stride >= 0 and a multiple of 8 elements
 *            (16 bytes); input strides may be 0 (a tensor shared across
 *            batches or heads).  Read during the call only.
 *   out      distinct (b, h, t) rows must not overlap, and the whole address
 *            range the output spans must not overlap the range of any input
 *            or of lambda
 *   other arguments as for diffattn_fwd; bf16 only
 * Errors: as diffattn_fwd, plus ERR_INVALID for a null `strides`, a negative
 * stride or overlapping output rows, ERR_UNSUPPORTED for fp32, a stride that
 * is not a multiple of 8, or a K1, K2 or V row stride that puts a row 2 GiB
 * or more past the start of its (b, h) slice.
 */
diffattn_status diffattn_fwd_strided(int dtype, int B, int H, int T, int D, const void* q1,
                                     const void* k1, const void* q2, const void* k2, const void* v,
                                     const long long* strides, const float* lambda, int causal,
                                     int headnorm, float lambda_init, float eps, void* out,
                                     hipStream_t stream);

/*
 * Prefill with a causal sliding window (the French lesson page, "Utilisez-le":
 * hybrid stacks that alternate differential attention with sliding-window
 * attention).  Row i sees the `window` most recent positions including itself,
 * keys j with i - window < j <= i, in both maps; a window of T or more is the
 * causal mask.  Key tiles outside every row's window are neither loaded nor
 * computed.
 *
 *   window          >= 1
 *   other arguments as for diffattn_fwd (causal implied); bf16 only
 * Errors: as diffattn_fwd, plus ERR_INVALID for window < 1 and
 * ERR_UNSUPPORTED for fp32.
 */
diffattn_status diffattn_fwd_window(int dtype, int B, int H, int T, int D, const void* q1,
                                    const void* k1, const void* q2, const void* k2, const void* v,
                                    const float* lambda, int window, int headnorm, float lambda_init,
                                    float eps, void* out, hipStream_t stream);

/*
 * Prefill forward with lambda formed in the same launch: exactly
 * diffattn_lambda(lq1, lk1, lq2, lk2, H, Dl, lambda_init, lambda) followed by
 * diffattn_fwd(..., lambda, ...), as one kernel (aifetchly page, section 3,
 * for lambda; paperleet page, equation for A1, A2, O, for the rest).  Every
 * workgroup forms the lambda of its head from the four vectors with the same
 * arithmetic as diffattn_lambda, so the result is identical bit for bit; the
 * separate lambda launch and its kernel boundary disappear.
 *
 *   q1 .. v, causal, headnorm, eps, out   as for diffattn_fwd
 *   lq1, lk1, lq2, lk2  device fp32 [H, Dl]
 *   lambda_init         added to lambda, and the (1 - lambda_init) head-norm
 *                       multiplier as in diffattn_fwd
 *   lambda_out          optional device fp32 [H] that receives lambda (NULL:
 *                       not written), e.g. for a decode call that follows
 * Errors: as diffattn_fwd, plus ERR_INVALID for a null vector, Dl < 1 or
 * lambda_out overlapping an input or out, and ERR_UNSUPPORTED for a vector or
 * lambda_out not 4-byte aligned.
 */
diffattn_status diffattn_fwd_reparam(int dtype, int B, int H, int T, int D, const void* q1,
                                     const void* k1, const void* q2, const void* k2,
                                     const void* v, const float* lq1, const float* lk1,
                                     const float* lq2, const float* lk2, int Dl, int causal,
                                     int headnorm, float lambda_init, float eps,
                                     float* lambda_out, void* out, hipStream_t stream);

/*
 * Standard softmax attention, softmax(Q K^T / sqrt(D) + M) V, bf16 only: the
 * comparison kernel for a differential head of the same size (a differential
 * head of width D/2 has the same parameter count and the same 8 (D/2) flops
 * per query-key pair; the glossary page compares the throughput of the two
 * kinds of model).  It is the lambda = 0 case of diffattn_fwd with one map,
 * and runs the same kernel with one score map.
 *
 *   q, k, v, out    [B, H, T, D] bf16, D = 64 or 128
 *   causal          as for diffattn_fwd
 * Errors: ERR_INVALID (null pointer, B/H/T < 1, out overlapping an input),
 * ERR_UNSUPPORTED (dtype other than bf16, D, alignment, grid size), ERR_HIP.
 */
diffattn_status diffattn_attention_fwd(int dtype, int B, int H, int T, int D, const void* q,
                                       const void* k, const void* v, int causal, void* out,
                                       hipStream_t stream);

/*
 * Number of key splits decode uses for (B, H, L) when num_splits = 0.
 */
int diffattn_decode_default_splits(int B, int H, int L);

/*
 * Bytes of fp32 workspace diffattn_decode needs: B*H*S*2*(2D+2)*4 with
 * S = num_splits, or the default split count when num_splits = 0.
 * Returns 0 for invalid sizes.
 */
size_t diffattn_decode_workspace_bytes(int B, int H, int L, int D, int num_splits);

/*
 * Decode: one new query per (b, h) against a KV cache of L rows, no mask
 * (the French lesson page "Attention différentielle (V2)", "V1 contre V2":
 * the value cache is read once per step for both maps).
 *
 *   q1, q2          [B, H, D]
 *   k1, k2          [B, H, L, D]   caches
 *   v               [B, H, L, 2D]  cache
 *   lambda          [H] fp32 (device)
 *   headnorm, lambda_init, eps   as for diffattn_fwd
 *   num_splits      number of key chunks (split-K), 1..L; 0 = default
 *   workspace       device scratch of at least
 *                   diffattn_decode_workspace_bytes(B, H, L, D, num_splits)
 *                   bytes, 16-byte aligned; its contents on entry are ignored
 *                   and calls on one stream may reuse it (calls that run
 *                   concurrently need separate workspaces)
 *   out             [B, H, 2D]
 * Errors: as diffattn_fwd, plus ERR_INVALID for num_splits < 0 or > L and
 * ERR_WORKSPACE for a null or too small workspace.
 */
diffattn_status diffattn_decode(int dtype, int B, int H, int L, int D, const void* q1,
                                const void* k1, const void* q2, const void* k2, const void* v,
                                const float* lambda, int headnorm, float lambda_init, float eps,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                void* out, hipStream_t stream);

/*
 * Decode over caches filled to different lengths per sequence (a serving
 * batch in which every sequence has its own context length): sequence b
 * attends to its first lengths[b] cached rows only.
 *
 *   lengths   [B] int32, DEVICE memory, each in [0, L] (values outside are
 *             clamped to that range, so no row past L is ever read); a length
 *             of 0 gives a zero output row (no key to attend to)
 *   other arguments as for diffattn_decode (L is the cache capacity, the
 *   row stride of k1, k2, v)
 * Errors: as diffattn_decode, plus ERR_INVALID for a null `lengths` or one
 * overlapping the output or workspace, ERR_UNSUPPORTED for a misaligned one.
 */
diffattn_status diffattn_decode_ragged(int dtype, int B, int H, int L, int D, const void* q1,
                                       const void* k1, const void* q2, const void* k2,
                                       const void* v, const float* lambda, const int* lengths,
                                       int headnorm, float lambda_init, float eps, int num_splits,
                                       void* workspace, size_t workspace_bytes, void* out,
                                       hipStream_t stream);

/*
 * Size in bytes of the device array diffattn_decode_noalloc works in (one per
 * GPU).
 */
#define DIFFATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * diffattn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc): the
 * same kernels and the same result bit for bit, but no workspace argument.
 * The split-K partial states go to a static device array of
 * DIFFATTN_NOALLOC_SCRATCH_BYTES bytes that the library holds, one copy per
 * GPU, from its load until the process ends.  The copy of the current device
 * (hipGetDevice) is used, so `stream` must belong to that device.  The first
 * call on a device looks up the array's device address
 * (hipGetSymbolAddress; to keep that lookup out of a graph capture, make one
 * call on each device before capturing).  No call allocates or frees memory.
 *
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * partial states: calls that can overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.  The array's contents on
 * entry are ignored, so nothing needs to be cleared between calls.
 *
 *   arguments as for diffattn_decode, without workspace and workspace_bytes
 * Errors: as diffattn_decode; ERR_WORKSPACE when
 * diffattn_decode_workspace_bytes(B, H, L, D, num_splits) exceeds
 * DIFFATTN_NOALLOC_SCRATCH_BYTES (fewer splits, or diffattn_decode with a
 * workspace of the caller's, then fit); ERR_HIP when the array's address
 * cannot be obtained (no device).
 */
diffattn_status diffattn_decode_noalloc(int dtype, int B, int H, int L, int D, const void* q1,
                                        const void* k1, const void* q2, const void* k2,
                                        const void* v, const float* lambda, int headnorm,
                                        float lambda_init, float eps, int num_splits, void* out,
                                        hipStream_t stream);

/*
 * ---- DIFF V2 (the French lesson page "Attention différentielle (V2)",
 *      "V1 contre V2") ----
 *
 * V2 doubles the query heads and keeps the baseline's KV heads and head
 * width: the two queries of differential head p read the same K and V (those
 * of KV head g = p / (H / Hkv), the grouping of grouped-query attention), the
 * difference is taken after attention, and there is no per-head norm:
 *
 *   O_p = (softmax(Q1_p K_g^T / sqrt(D) + M) - lambda_p softmax(Q2_p K_g^T / sqrt(D) + M)) V_g
 *
 * bf16 only, D = 64 or 128, fp32 accumulation; mask and lambda as for
 * diffattn_fwd.
 *
 *   q1, q2   [B, H, T, D]    the two query heads of each differential head
 *   k, v     [B, Hkv, T, D]  H must be a whole multiple of Hkv
 *   lambda   [H] fp32 (device)
 *   out      [B, H, T, D]
 * Errors: ERR_INVALID (null pointer, sizes < 1, H not a multiple of Hkv,
 * overlapping output), ERR_UNSUPPORTED (dtype other than bf16, D, alignment,
 * grid size), ERR_HIP.
 */
diffattn_status diffattn_v2_fwd(int dtype, int B, int H, int Hkv, int T, int D, const void* q1,
                                const void* q2, const void* k, const void* v, const float* lambda,
                                int causal, void* out, hipStream_t stream);

/*
 * Bytes of fp32 workspace diffattn_v2_decode needs: B*H*S*2*(D+2)*4, with
 * S = num_splits or, for num_splits = 0, diffattn_decode_default_splits(B, Hkv, L).
 * Returns 0 for invalid sizes.
 */
size_t diffattn_v2_decode_workspace_bytes(int B, int H, int Hkv, int L, int D, int num_splits);

/*
 * V2 decode: one new query pair per (b, differential head) against the KV
 * cache of its group, no mask.  Each workgroup reads a chunk of one KV head's
 * cache once and serves all H / Hkv differential heads of the group (both
 * maps of each), so the cache bytes per step are those of a grouped-query
 * baseline with the same (Hkv, H).
 *
 *   q1, q2   [B, H, D]
 *   k, v     [B, Hkv, L, D]  caches; H / Hkv must be 1, 2 or 4
 *   lambda   [H] fp32 (device)
 *   num_splits, workspace, workspace_bytes   as for diffattn_decode (sized by
 *            diffattn_v2_decode_workspace_bytes)
 *   out      [B, H, D]
 * Errors: as diffattn_v2_fwd, plus ERR_INVALID for num_splits < 0 or > L,
 * ERR_UNSUPPORTED for another group size, ERR_WORKSPACE for a null or too
 * small workspace.
 */
diffattn_status diffattn_v2_decode(int dtype, int B, int H, int Hkv, int L, int D, const void* q1,
                                   const void* q2, const void* k, const void* v, const float* lambda,
                                   int num_splits, void* workspace, size_t workspace_bytes, void* out,
                                   hipStream_t stream);

/*
 * ---- Training: forward with saved state, and the backward pass ----
 *
 * The paperleet page "Differential Transformer Attention" asks for gradients
 * through both Q/K branches, the value and the coefficient lambda, and
 * through the four re-parameterisation vectors of lambda.  These entry points
 * support bf16 tensors with D = 32, 64 or 128.
 *
 * Bytes of the saved-state buffer diffattn_fwd_train fills and diffattn_bwd
 * reads: 2 * B*H*T*2D*4 + B*H*2*T*4 (fp32 per-map outputs A1 V and A2 V, then
 * each map's log2-domain log-sum-exp of its scaled scores per row, layout
 * [B,H,2,T]).  Returns 0 for unsupported sizes.
 */
size_t diffattn_train_saved_bytes(int B, int H, int T, int D);

/*
 * diffattn_fwd (same arguments and output, bf16 only, D = 32, 64 or 128) that also
 * writes the saved state the backward pass needs into `saved` (at least
 * diffattn_train_saved_bytes bytes, 16-byte aligned, disjoint from every
 * input and from out).  The output is identical to diffattn_fwd's.
 * Errors: as diffattn_fwd; ERR_UNSUPPORTED for fp32 or D other than 32, 64, 128;
 * ERR_WORKSPACE when saved_bytes is too small.
 */
diffattn_status diffattn_fwd_train(int dtype, int B, int H, int T, int D, const void* q1,
                                   const void* k1, const void* q2, const void* k2, const void* v,
                                   const float* lambda, int causal, int headnorm, float lambda_init,
                                   float eps, void* out, void* saved, size_t saved_bytes,
                                   hipStream_t stream);

/*
 * Bytes of device workspace diffattn_bwd needs (16-byte aligned): the
 * gradient reaching the pre-norm output (bf16 [B,H,T,2D]), per-row
 * statistics (fp32 [B,H,4,Tp], Tp = T rounded up to 64) and per-chunk
 * partial sums of dlambda (fp32 [B,H,Tp/64]).  Returns 0 for unsupported
 * sizes.
 */
size_t diffattn_bwd_workspace_bytes(int B, int H, int T, int D);

/*
 * Backward pass of diffattn_fwd_train: given dL/dout, the gradients
 *   dq1, dk1, dq2, dk2  [B, H, T, D]   bf16
 *   dv                  [B, H, T, 2D]  bf16
 *   dlambda             [H] fp32: dL/dlambda_h summed over batch and tokens
 * and, when the four re-parameterisation vectors lq1, lk1, lq2, lk2 ([H, Dl]
 * fp32, those lambda was formed from with diffattn_lambda) are given, their
 * gradients dlq1, dlk1, dlq2, dlk2 ([H, Dl] fp32), by the chain rule through
 * lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init (aifetchly page,
 * section 3).  Pass all eight vector pointers or none.
 *
 *   q1 .. v, lambda, causal, headnorm, lambda_init, eps
 *                 exactly as given to diffattn_fwd_train
 *   dout          [B, H, T, 2D] bf16, gradient of the forward's output
 *   saved         the buffer diffattn_fwd_train filled (read only)
 *   workspace     device scratch of at least diffattn_bwd_workspace_bytes;
 *                 contents on entry ignored; concurrent calls need separate
 *                 workspaces
 * The maps are recomputed from the saved log-sum-exp, never stored.  dlambda
 * and the vector gradients are summed in a fixed order (deterministic).
 * Errors: ERR_INVALID (null tensor pointer, B/H/T < 1, headnorm with eps <= 0,
 * only some of the vector pointers, Dl < 1 with vectors, any output
 * overlapping an input, another output or the workspace), ERR_UNSUPPORTED
 * (dtype other than bf16, D other than 32, 64 or 128, misalignment, sizes),
 * ERR_WORKSPACE (saved_bytes or workspace too small), ERR_HIP.
 */
diffattn_status diffattn_bwd(int dtype, int B, int H, int T, int D, const void* q1, const void* k1,
                             const void* q2, const void* k2, const void* v, const float* lambda,
                             const void* dout, const void* saved, size_t saved_bytes, int causal,
                             int headnorm, float lambda_init, float eps, void* dq1, void* dk1,
                             void* dq2, void* dk2, void* dv, float* dlambda, const float* lq1,
                             const float* lk1, const float* lq2, const float* lk2, int Dl,
                             float* dlq1, float* dlk1, float* dlq2, float* dlk2, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
