/*
 * qkv.h -- C ABI of the fused attention-input library for AMD Instinct MI355X (gfx950).
 *
 * One call computes, for T tokens, the attention-input chain of a Llama-style
 * decoder layer:
 *
 *     r[t]   = 1 / sqrt( (1/H) * sum_k x[t,k]^2 + eps )              (RMSNorm row reduction)
 *     a[t,k] = x[t,k] * r[t] * w_norm[k]                             (normalised activations)
 *     y[t,n] = sum_k a[t,k] * W[k,n]  (+ bias[n])                    (QKV projection)
 *     Q, K   = rotate-half rotary embedding of the Q and K heads of y at position pos[t]
 *     V      = the V heads of y, unrotated
 *
 * The chain is the one the page "Liger-Kernel底层优化：新一代内核级推理加速引擎介绍"
 * (Liger-Kernel low-level optimisation: a new kernel-level inference acceleration
 * engine) lists for one decoder layer in its opening section (rms_norm, proj_qkv,
 * apply_rope on q and on k), and that the same page's section
 * "融合内核是如何工作的？来看一段简化版实现" (how the fused kernel works) sketches as
 * a single fused kernel: eps inside the reciprocal square root over the mean of
 * squares, the weight multiplying each normalised element, the bias added before
 * the rotation, and feature i of a head paired with feature i + head_dim/2.
 * The rotation turns each pair (u, v) by +phi, phi = pos * theta^(-2i/head_dim):
 *     (u, v) -> (u*cos(phi) - v*sin(phi), v*cos(phi) + u*sin(phi)).
 *
 * Layouts (all dense, row-major, no strides):
 *     x      [T, H]                 dtype of the plan
 *     w_norm [H]                    dtype of the plan
 *     w_qkv  [H, N]                 dtype of the plan; N = (nq + 2*nkv) * head_dim;
 *                                   columns = Q heads | K heads | V heads, each head's
 *                                   head_dim columns contiguous
 *     bias   [N] or NULL            dtype of the plan
 *     pos    [T] int32              position id of each token (any int32 value)
 *     q      [T, nq*head_dim]       written, dtype of the plan
 *     k, v   [T, nkv*head_dim]      written, dtype of the plan
 *
 * Precision: bf16 plans take bf16 inputs and write bf16 outputs (round to nearest
 * even); products accumulate in fp32.  fp32 plans compute in fp32 throughout.
 *
 * Ownership: the caller owns every tensor, allocates the outputs, and keeps all
 * buffers alive until the work queued on `stream` has finished.  A plan owns only
 * its device scratch (per-token inverse RMS values, decode partial sums and
 * counters, the split-K prefill form's partial tiles -- up to 67 MB -- and counters,
 * the rotary frequency table, and with QKV_PLAN_PREFILL_PREPASS the pre-pass's bf16
 * products -- ceil(max_tokens / 256) * 256 * hidden * 2 bytes), allocated on the
 * device that is current when the plan is created and freed by qkv_plan_destroy.
 *
 * Errors: every call returns a status code; nothing is thrown across the ABI.
 * Arguments are validated before any HIP call is made.
 */
#ifndef QKV_MI355X_H
#define QKV_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qkv_status {
  QKV_OK = 0,
  QKV_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, malformed descriptor */
  QKV_ERR_UNSUPPORTED = 2,   /* well-formed request outside what the kernels implement  */
  QKV_ERR_HIP = 3,           /* a HIP runtime call or kernel launch failed              */
  QKV_ERR_OUT_OF_MEMORY = 4  /* device scratch allocation failed                        */
} qkv_status;

typedef enum qkv_dtype {
  QKV_F32 = 0,
  QKV_BF16 = 1
} qkv_dtype;

/* Kernel path a forward of a given token count runs on (see qkv_plan_variant). */
typedef enum qkv_variant {
  QKV_VARIANT_GENERIC = 0,  /* fp32 FMA tiles: any supported shape, both dtypes        */
  QKV_VARIANT_PREFILL = 1,  /* one bf16 MFMA launch normalising the activations as
                               they are loaded, applying 1/rms, bias and rotation
                               (two launches with QKV_PLAN_PREFILL_PREPASS)             */
  QKV_VARIANT_DECODE = 2,   /* bf16 MFMA weight-streaming kernel for small token counts:
                               up to 192 (or 256) tokens, one launch per 128 tokens     */
  QKV_VARIANT_PREFILL_SPLIT = 3  /* the prefill kernel with the hidden dimension split over
                               two workgroups per tile, when the tiles alone would leave
                               at least half of the CUs idle                            */
} qkv_variant;

typedef struct qkv_plan_s* qkv_plan;

typedef struct qkv_plan_desc {
  int64_t max_tokens;     /* upper bound on T for every forward through this plan (>= 1) */
  int32_t hidden;         /* H: multiple of 8                                            */
  int32_t num_q_heads;    /* nq >= 1                                                     */
  int32_t num_kv_heads;   /* nkv >= 1, nq % nkv == 0 (MHA when equal, GQA otherwise)     */
  int32_t head_dim;       /* even; the kernels implement multiples of 8                  */
  int32_t dtype;          /* qkv_dtype                                                   */
  int32_t has_bias;       /* 0 or 1                                                      */
  double eps;             /* >= 0, finite; added to the mean square inside the sqrt      */
  double rope_theta;      /* > 0, finite; rotary base                                    */
  int32_t flags;          /* 0, or QKV_PLAN_PREFILL_PREPASS                              */
} qkv_plan_desc;

/* Plan flag: plain prefill forwards (QKV_VARIANT_PREFILL) run as two launches, a pre-pass
 * that writes bf16(x * w_norm) and each row's 1/rms to plan scratch
 * (ceil(max_tokens / 256) * 256 * hidden * 2 bytes, allocated at plan creation), then the
 * 256 x 256 MFMA kernel streaming those activations from HBM.  Without the flag (the
 * default) the normalised activations never leave the chip: one launch normalises each
 * row as it is loaded.  The flag exists to measure the trade-off; results agree within
 * the parity bar, not bit for bit. */
#define QKV_PLAN_PREFILL_PREPASS 1

/* Validate `desc`, pick the kernel variants, allocate the plan's device scratch on
 * the current device and return an opaque handle in *out_plan.
 * Returns QKV_ERR_INVALID_ARG for a malformed descriptor or null pointers,
 * QKV_ERR_UNSUPPORTED for shapes outside the kernels (head_dim not a multiple of 8,
 * tensors whose byte size reaches 2^31, with QKV_PLAN_PREFILL_PREPASS also a pre-pass
 * buffer of 2^31 bytes or more), QKV_ERR_HIP when no device is usable and
 * QKV_ERR_OUT_OF_MEMORY when the scratch cannot be allocated.  On error *out_plan is
 * left NULL. */
qkv_status qkv_plan_create(const qkv_plan_desc* desc, qkv_plan* out_plan);

/* Queue one forward of T = num_tokens tokens on `stream` (a hipStream_t; NULL is the
 * null stream).  Asynchronous: returns once the kernels are queued; allocates
 * nothing and never synchronises the host.  T == 0 is a no-op that returns QKV_OK
 * without touching any pointer.  For T >= 1: every pointer except `bias` must be
 * non-null; `bias` must be non-null exactly when the plan has has_bias = 1; x,
 * w_norm, w_qkv, bias, q, k and v must be 16-byte aligned and pos 4-byte aligned;
 * 1 <= T <= max_tokens.  Violations return QKV_ERR_INVALID_ARG before anything is
 * queued.  The device current at the call must be the plan's device.
 * Forwards through the same plan share its scratch: two forwards through one plan
 * on different streams may not overlap in time (use one plan per stream).
 * Launch failures return QKV_ERR_HIP. */
qkv_status qkv_forward(qkv_plan plan, int64_t num_tokens,
                       const void* x, const void* w_norm, const void* w_qkv,
                       const void* bias, const int32_t* pos,
                       void* q, void* k, void* v, void* stream);

/* The same forward with K and V written into key/value caches instead of dense
 * buffers: the K row and the V row of token t (nkv*head_dim elements each, dtype of
 * the plan) go to row slots[t] of k_cache and of v_cache, both dense
 * [cache_rows, nkv*head_dim]; Q is written densely as in qkv_forward.  This is the
 * step that follows the chain in generation: the new keys and values appended to the
 * preallocated, fixed-size cache of the RollingBuffer part of the page
 * "Liger-Kernel内核级优化：FlashAttention与RollingBuffer详解" (Liger-Kernel
 * kernel-level optimisation: FlashAttention and RollingBuffer explained), which
 * reuses the cache circularly: a rolling cache of capacity C for one sequence takes
 * slots[t] = pos[t] mod C (plus the sequence's first row when several sequences share
 * one buffer).  Here the caller chooses the slots, so contiguous, paged and rolling
 * caches all use this one call.
 * slots: [T] int32, 4-byte aligned.  A token whose slot lies outside [0, cache_rows)
 * (for instance -1 for padding) writes no K and V; rows that no slot names are left
 * untouched.  Two tokens of one call must not name the same slot (which of them
 * lands is then unspecified).  k_cache and v_cache must be 16-byte aligned and
 * cache_rows >= 1; a cache of 2^31 bytes or more returns QKV_ERR_UNSUPPORTED.
 * Everything else (other arguments, asynchrony, scratch sharing, errors) is as for
 * qkv_forward. */
qkv_status qkv_forward_kv_cache(qkv_plan plan, int64_t num_tokens,
                                const void* x, const void* w_norm, const void* w_qkv,
                                const void* bias, const int32_t* pos,
                                const int32_t* slots, int64_t cache_rows,
                                void* q, void* k_cache, void* v_cache, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc: the forward of qkv_forward
 * without a plan.  `desc` describes the layer exactly as for qkv_plan_create
 * (validated the same way; T = num_tokens must satisfy 1 <= T <= desc->max_tokens;
 * desc->flags must be 0, since the pre-pass form needs plan scratch, else
 * QKV_ERR_UNSUPPORTED), and every other argument is as for qkv_forward.  Nothing is allocated: the call's
 * scratch (its rotary table and the decode kernel's partial sums and arrival counters)
 * lives in one file-scope device array of the library, 16,912,384 bytes per GPU,
 * reserved on every GPU the library runs on until the process ends.  Each call first
 * queues a one-workgroup kernel that writes its rotary table and zeroes the counters,
 * then the forward's kernels: the decode kernel for up to 256 tokens (consecutive
 * launches of up to 128) on shapes it supports, else the single-launch
 * normalise-on-load prefill kernel (never its split-K form, whose partial tiles would
 * not fit), else the generic kernel; results match qkv_forward's within the same
 * tolerance (bit for bit where both run the same kernel).
 * All calls on one GPU share that array: two calls that overlap in time on one GPU
 * (different streams, or different host threads on one stream without ordering) race
 * and may return wrong results; queue them on one stream, one after the other.
 * head_dim above 512 (a table beyond the array's slot) returns QKV_ERR_UNSUPPORTED;
 * argument errors return QKV_ERR_INVALID_ARG before any HIP call; a failed launch or
 * symbol lookup returns QKV_ERR_HIP. */
qkv_status qkv_forward_noalloc(const qkv_plan_desc* desc, int64_t num_tokens,
                               const void* x, const void* w_norm, const void* w_qkv,
                               const void* bias, const int32_t* pos,
                               void* q, void* k, void* v, void* stream);

/* Queue only the row reduction of the chain: inv_rms[t] = 1/sqrt(mean_k x[t,k]^2 + eps)
 * as fp32 for t < num_tokens, into the caller's device buffer `inv_rms` (4-byte
 * aligned).  Same argument rules, asynchrony and errors as qkv_forward. */
qkv_status qkv_rms_inv(qkv_plan plan, int64_t num_tokens, const void* x,
                       float* inv_rms, void* stream);

/* The chain's steps unfused, for measuring what the fusion saves.  The pages on
 * Liger-Kernel credit fusing RMSNorm, the projection and RoPE with fewer launches and
 * fewer HBM round trips (page "Liger-Kernel底层优化：新一代内核级推理加速引擎介绍", the
 * sections on why fusion pays and on the fused kernel).  These entry points run the same arithmetic as
 * separate kernels, each reading its input from and writing its output to HBM.
 * Same plan, argument rules (dtype, alignment to 16 bytes, 4 for pos), asynchrony and
 * errors as qkv_forward.
 *
 * qkv_rms_norm: xn [T, H] = x[t,k] * 1/sqrt(mean_k x[t,k]^2 + eps) * w_norm[k] (the
 *   fused chain's normalised activations, computed in fp32, rounded once to the plan
 *   dtype), into the caller's buffer xn. */
qkv_status qkv_rms_norm(qkv_plan plan, int64_t num_tokens, const void* x, const void* w_norm,
                        void* xn, void* stream);

/* qkv_rope: in place on a projection output y [T, N] laid out like the fused forward's
 * outputs side by side (columns: the Q heads, then K, then V): adds bias [N] to every
 * column (exactly when the plan has has_bias = 1; NULL otherwise), then turns each
 * rotate-half pair (i, i + head_dim/2) of every Q and K head by pos[t] * theta^(-2i/d)
 * radians, as the fused forward does; V gets only the bias. */
qkv_status qkv_rope(qkv_plan plan, int64_t num_tokens, const void* bias, const int32_t* pos,
                    void* y, void* stream);

/* qkv_head_norm_rope: a norm and the rotation in one pass, in place on y [T, N] laid out
 * as for qkv_rope.  The Liger-Kernel pages name a fused RMSNorm + RoPE operator without
 * defining it; in this chain the two are not adjacent, so it is read as the one form in
 * which they are: every Q head divided by its own RMS over its head_dim values (eps of
 * the plan) and multiplied by w_qnorm [head_dim], every K head likewise with w_knorm
 * [head_dim], then each head's rotate-half pairs turned as in qkv_rope; V untouched.
 * Arithmetic in fp32, one rounding to the plan dtype.  head_dim above 256 returns
 * QKV_ERR_UNSUPPORTED; otherwise as qkv_rope. */
qkv_status qkv_head_norm_rope(qkv_plan plan, int64_t num_tokens, const void* w_qnorm,
                              const void* w_knorm, const int32_t* pos, void* y, void* stream);

/* qkv_forward_unfused: the whole chain as three steps -- qkv_rms_norm into the caller's
 * xn [T, H], the projection y = xn W_qkv as a rocBLAS GEMM (fp32 accumulation, output in
 * the plan dtype) into the caller's y [T, N], then qkv_rope on y.  Q, K and V are the
 * column blocks [0, nq*d), [nq*d, (nq+nkv)*d) and the rest of y.  Each step rounds its
 * output to the plan dtype, so results differ from qkv_forward's by those roundings.
 * The first call on a plan creates its GEMM library handle (host allocation and device
 * memory; not under graph capture). */
qkv_status qkv_forward_unfused(qkv_plan plan, int64_t num_tokens,
                               const void* x, const void* w_norm, const void* w_qkv,
                               const void* bias, const int32_t* pos,
                               void* xn, void* y, void* stream);

/* Backward of the chain: given the gradients dq [T, nq*head_dim], dk and dv
 * [T, nkv*head_dim] of a loss with respect to Q, K and V, write its gradients with
 * respect to the inputs:
 *     dx       [T, H]   (overwritten)
 *     dw_norm  [H]      (overwritten, summed over the T tokens)
 *     dw_qkv   [H, N]   (overwritten, summed over the T tokens)
 *     dbias    [N]      (overwritten, summed over the T tokens) -- exactly when the
 *                       plan has has_bias = 1, NULL otherwise
 * all in the plan dtype, for the same x, w_norm, w_qkv and pos as the forward (the
 * bias value does not enter the gradients).  The chain rule, step by step: each
 * (dq, dk) pair is turned back by -angle (the transpose of the rotation), the bias
 * gradient is the column sum of that, dW = a^T gy and ga = gy W^T with a = x r w the
 * normalised activations (recomputed), dw_norm = sum_t ga x r, and
 * dx_j = r w_j ga_j - (r^3/H) x_j sum_k ga_k w_k x_k.  The page
 * "Liger-Kernel核心技术：RollingBuffer与融合算子详解" reports backward speed-ups for its
 * fused kernels next to the forward ones (section "算子融合").
 * The normalised activations are never formed: r scales the unrotated gradient
 * (g = r gy, rounded once to the plan dtype), so that dW = diag(w) x^T g with x itself
 * as the GEMM operand, G = g W^T = r ga, db = sum_t g / r, dw_norm = sum_t G x and
 * dx_j = w_j G_j - (r^2/H) x_j sum_k G_k w_k x_k -- the same algebra.
 * Every step, the two products included, runs on this library's kernels: for bf16
 * plans both GEMMs on the matrix cores (bf16 operands, fp32 accumulation; G = g W^T
 * there when N is a multiple of 32, else on fp32 FMA tiles), for fp32 plans on fp32
 * FMA tiles.  dW and the intermediate G are rounded once to the plan dtype from their
 * fp32 results.
 * Column sums are done in a fixed order and every GEMM element is one fixed-order
 * sum, so results are deterministic.
 * Scratch: the first backward call through a plan allocates the plan's backward
 * scratch (about max_tokens * (N + H) * e + 8192 H bytes, e = element size), kept until
 * qkv_plan_destroy; later calls allocate nothing.  Forwards and backwards through one
 * plan share scratch and must not overlap in time.
 * Limits: ceil(num_tokens / 32) * 32 * N * e < 2^31 (the transposed upstream gradient
 * is addressed with 32-bit byte offsets), else QKV_ERR_UNSUPPORTED.
 * Alignment: every tensor 16-byte aligned except pos (4 bytes).  num_tokens == 0 is a
 * no-op.  Argument errors return QKV_ERR_INVALID_ARG before any HIP call; failed
 * scratch allocation QKV_ERR_OUT_OF_MEMORY; launch failures QKV_ERR_HIP. */
qkv_status qkv_backward(qkv_plan plan, int64_t num_tokens,
                        const void* x, const void* w_norm, const void* w_qkv, const int32_t* pos,
                        const void* dq, const void* dk, const void* dv,
                        void* dx, void* dw_norm, void* dw_qkv, void* dbias, void* stream);

/* Gated MLP of the same decoder layer on the same normalise-on-load kernel:
 *
 *     r[t]     = 1 / sqrt( (1/H) * sum_k x[t,k]^2 + eps )
 *     a[t,k]   = x[t,k] * r[t] * w_norm[k]
 *     g, u     = a @ W_gate, a @ W_up          (W_gate_up = [W_gate | W_up], [H, 2I])
 *     out[t,j] = SiLU(g[t,j]) * u[t,j],  SiLU(z) = z / (1 + exp(-z))
 *
 * The fused linear SwiGLU of the operator-fusion section ("算子融合") of the page
 * "Liger-Kernel核心技术：RollingBuffer与融合算子详解" (Liger-Kernel core techniques:
 * RollingBuffer and fused operators explained): both products of one input against
 * the gate and up weights, the SiLU and the elementwise product done in registers,
 * only the result written; preceded here by the layer's RMSNorm, exactly as in
 * qkv_forward.  No bias.
 * Layouts (dense, row-major): x [T, H], w_norm [H], w_gate_up [H, 2I] with the gate
 * columns first, out [T, I]; all 16-byte aligned.  Stateless: no plan, nothing
 * allocated, asynchronous on `stream`; runs on the current device.
 * bf16 only (dtype = QKV_BF16), H and I multiples of 128, and each of x, w_gate_up
 * and out under 2^31 bytes; other shapes or QKV_F32 return QKV_ERR_UNSUPPORTED.
 * num_tokens == 0 is a no-op; negative sizes, a bad dtype code, eps negative or not
 * finite, null or misaligned pointers return QKV_ERR_INVALID_ARG before any HIP call;
 * a failed launch returns QKV_ERR_HIP. */
qkv_status qkv_swiglu_forward(int64_t num_tokens, int32_t hidden, int32_t intermediate,
                              int32_t dtype, double eps,
                              const void* x, const void* w_norm, const void* w_gate_up,
                              void* out, void* stream);

/* Which variant a forward of num_tokens tokens runs on, in *variant (a qkv_variant):
 * bf16 plans of a shape the decode kernel supports take it up to 192 tokens, or up to
 * 256 when the prefill kernel has no split form for T (as consecutive launches of up
 * to 128 tokens, queued in order on the forward's stream); other bf16 plans of a
 * supported shape take the prefill kernel -- in its split form
 * (QKV_VARIANT_PREFILL_SPLIT) when T's 256 x 256 tiles number at most 128 and the
 * hidden size divides into two slices of a multiple of 4 steps of 32, at least 8 --
 * everything else generic.
 * Host-only; returns QKV_ERR_INVALID_ARG for a bad plan or num_tokens out of range. */
qkv_status qkv_plan_variant(qkv_plan plan, int64_t num_tokens, int32_t* variant);

/* Release the plan's scratch and the handle.  NULL is a no-op returning QKV_OK.
 * Waits for the plan's device to finish queued work before freeing.  A handle that
 * was already destroyed is detected on a best-effort basis (QKV_ERR_INVALID_ARG). */
qkv_status qkv_plan_destroy(qkv_plan plan);

/* Static, NUL-terminated description of a status code ("unknown status" otherwise). */
const char* qkv_status_string(qkv_status status);

/* Static name of a variant ("generic", "prefill", "decode", "prefill_split"; "unknown"
 * otherwise). */
const char* qkv_variant_name(int32_t variant);

#ifdef __cplusplus
}
#endif

#endif /* QKV_MI355X_H */
