/*
 * mt.h -- C ABI of one tensor-parallel (TP) shard of a GPT transformer layer,
 * forward and backward, on one AMD Instinct MI355X (gfx950).
 *
 * What the shard computes (pre-LN GPT layer; one rank of a t-way tensor-parallel group):
 *   U = LN1(X)
 *   QKV_i = U W_qkv_i^T + b_qkv_i          column-parallel: this rank's heads
 *   ctx_i = causal softmax attention over the rank's heads (scale 1/sqrt(d))
 *   O_i = ctx_i W_o_i^T                   row-parallel: a PARTIAL sum
 *   X2 = X + AR(O_i) + b_o;  V2 = LN2(X2)
 *   A_i = V2 W1_i^T + b1_i;  Z_i = GeLU(A_i)   (fused bias + GeLU epilogue)
 *   Y_i = Z_i W2_i^T                       row-parallel: a PARTIAL sum
 *   Out = X2 + AR(Y_i) + b_fc2
 * The block structure Y = f(X A) B with A split by columns and B split by rows, each
 * rank computing f(X A_i) B_i whose sum over ranks an all-reduce forms, and the split of
 * attention heads over ranks, follow the "Megatron-LM" concept report
 * (compassingai.com), section 4.1; communication in the backward pass as well
 * (so the input-gradients of the column-parallel GEMMs are partials too) follows its
 * section 4.2. AR is the all-reduce point: on one GPU it is the identity, so for
 * tp > 1 the shard returns exactly what one rank computes before communicating; the
 * mt_mlp_* calls return the bare partials, whose sum over the t shards is the
 * unsharded block.
 *
 * Conventions for every call:
 *   - Device pointers are caller-owned, contiguous row-major, 16-byte aligned. The
 *     library allocates nothing and keeps no state between calls (apart from the
 *     optional timing records below).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). All work
 *     is enqueued asynchronously on it; faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - Activations and weights have the shape's dtype (MT_BF16: bfloat16 storage with
 *     fp32 accumulation and fp32 LayerNorm/softmax/GeLU math; MT_FP32: fp32 throughout;
 *     MT_BF16_QK: as MT_BF16, with the attention logits formed from Q and K carried as
 *     bf16 hi + lo pairs, see below).
 *     Parameter gradients are always fp32 and are overwritten (not accumulated).
 *   - Every argument is validated before anything is launched; on error nothing is
 *     launched and the status says why (mt_status_string).
 *   - Shape limits: h % heads == 0, heads % tp == 0, 0 <= shard < tp, head dim
 *     d = h / heads a multiple of 8, seq a multiple of 8 and <= 4096, h <= 32768.
 *   - Precision of the bf16 path: the residual stream X2 = X + O + b_o is kept in fp32
 *     inside the call; everything else stored between kernels (U, QKV, P, ctx, V2, A, Z,
 *     dA, dX2, dctx, dS, dQKV, partials) is bf16, each formed in fp32 and rounded once.
 *     db_o is summed from the unrounded dX2 where the LayerNorm-2 backward carries the
 *     column sums (h <= 16384), else from the stored dX2.
 *   - MT_BF16_QK: the softmax's exponent magnifies errors of the logits Q K^T / sqrt(d)
 *     by their own size, and with bf16 Q and K (8 significant bits) a shard whose logits
 *     reach the tens can miss the 2e-2 normwise bar on the attention gradients. In this
 *     mode LayerNorm 1 also writes the rounding remainder U_lo of U, the Q and K
 *     columns of the projection take (U + U_lo) W^T and are stored as hi + lo bf16
 *     pairs, and the logits are Q_hi K_hi^T + Q_hi K_lo^T + Q_lo K_hi^T (Q and K to
 *     about 16 bits). Cost: one more GEMM over the Q and K columns, two more logit
 *     products, and the remainders in the saved store and workspace.
 *   - Attention of the bf16 paths with head dim 64, 128 or 160 is fused: the logits and
 *     probabilities stay on chip, the saved store keeps each row's log-sum-exp (fp32)
 *     (and under MT_BF16_QK the Q, K remainders) instead of P, and the backward
 *     recomputes P. Other head dims, and the fp32 path, store P and the gradients of
 *     the logits.
 */
#ifndef MT_H_
#define MT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MT_OK = 0,
  MT_ERR_INVALID_ARG = 1, /* null pointer, misalignment, inconsistent shape */
  MT_ERR_UNSUPPORTED = 2, /* valid shape outside the supported limits above */
  MT_ERR_HIP = 3,         /* a HIP launch or runtime call failed */
  MT_ERR_WORKSPACE = 4,   /* saved / workspace buffer smaller than the *_bytes query */
  MT_ERR_NOALLOC_LIMIT = 5 /* mt_mlp_bwd_noalloc: the shape's scratch exceeds MT_NOALLOC_SCRATCH_BYTES */
} mt_status;

typedef enum { MT_BF16 = 0, MT_FP32 = 1, MT_BF16_QK = 2 } mt_dtype;

/* One TP shard of one layer. h and heads are the GLOBAL (unsharded) sizes; the shard
 * owns heads/tp heads and 4h/tp FFN columns. */
typedef struct {
  int32_t h, heads, seq, micro_batch, tp, shard;
  int32_t dtype; /* mt_dtype */
} mt_shape;

/* Shard-local weights in nn.Linear layout W[out, in], dtype of the shape.
 * M = micro_batch * seq tokens, ht = h/tp, ft = 4h/tp. */
typedef struct {
  const void *ln1_g, *ln1_b; /* [h] */
  const void *w_qkv;         /* [3*ht, h]: rows = [Q heads | K heads | V heads] of the shard */
  const void *b_qkv;         /* [3*ht] */
  const void *w_o;           /* [h, ht] */
  const void *b_o;           /* [h] replicated; added after the all-reduce point */
  const void *ln2_g, *ln2_b; /* [h] */
  const void *w_fc1;         /* [ft, h] */
  const void *b_fc1;         /* [ft] */
  const void *w_fc2;         /* [h, ft] */
  const void *b_fc2;         /* [h] replicated */
} mt_layer_weights;

/* fp32 parameter gradients, same shapes as mt_layer_weights. The replicated ones
 * (LayerNorm, b_o, b_fc2) are this rank's copy. */
typedef struct {
  float *ln1_g, *ln1_b, *w_qkv, *b_qkv, *w_o, *b_o, *ln2_g, *ln2_b, *w_fc1, *b_fc1, *w_fc2, *b_fc2;
} mt_layer_grads;

/* Bytes of the activation store written by mt_layer_fwd and read by mt_layer_bwd, and
 * of the scratch workspace either call needs (no initialisation required). Return 0
 * for an invalid shape. */
size_t mt_layer_saved_bytes(const mt_shape *shape);
size_t mt_layer_workspace_bytes(const mt_shape *shape);

/* Forward of the shard: x [M, h] -> out [M, h]. `saved` must stay untouched until the
 * matching mt_layer_bwd has run. */
int mt_layer_fwd(const mt_shape *shape, const mt_layer_weights *w, const void *x, void *out, void *saved,
                 size_t saved_bytes, void *workspace, size_t workspace_bytes, void *stream);

/* Backward of the shard given dout [M, h]: writes dx [M, h] (activation dtype) and every
 * parameter gradient in `grads` (fp32). x and w must be those of the forward. */
int mt_layer_bwd(const mt_shape *shape, const mt_layer_weights *w, const void *x, const void *saved,
                 size_t saved_bytes, const void *dout, void *dx, const mt_layer_grads *grads, void *workspace,
                 size_t workspace_bytes, void *stream);

/* MLP block alone, the concept report's f(X A_i) B_i (section 4.1):
 *   y_partial = GeLU(x W1^T + b1) W2^T  with x [M, h], W1 [ft, h], b1 [ft], W2 [h, ft].
 * No LayerNorm, no output bias, no residual: the sum of y_partial over the tp shards is
 * the unsharded block. */
size_t mt_mlp_saved_bytes(const mt_shape *shape);
size_t mt_mlp_workspace_bytes(const mt_shape *shape);
int mt_mlp_fwd(const mt_shape *shape, const void *x, const void *w_fc1, const void *b_fc1, const void *w_fc2,
               void *y_partial, void *saved, size_t saved_bytes, void *workspace, size_t workspace_bytes,
               void *stream);
/* Backward given dy [M, h]: dx_partial [M, h] (activation dtype; its sum over shards is
 * the block's input gradient, section 4.2), dw_fc1 [ft, h], db_fc1 [ft], dw_fc2 [h, ft]
 * in fp32. */
int mt_mlp_bwd(const mt_shape *shape, const void *x, const void *w_fc1, const void *w_fc2, const void *saved,
               size_t saved_bytes, const void *dy, void *dx_partial, float *dw_fc1, float *db_fc1, float *dw_fc2,
               void *workspace, size_t workspace_bytes, void *stream);

/* mt_mlp_bwd for callers that cannot allocate device memory (code being captured into
 * a HIP graph, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, the same kernels and bit-identical results. The
 * scratch those kernels need (the dA tile buffer and the column-sum partials,
 * mt_mlp_workspace_bytes(shape) bytes) comes from a static device array of
 * MT_NOALLOC_SCRATCH_BYTES inside the library: the HIP runtime allocates it on each
 * device when it loads the library's code there, and it is held until the process
 * ends. The call allocates nothing itself (no hipMalloc/hipFree, no events: per-launch
 * timing is skipped for it). Its first call on a device looks up that device's copy of
 * the array (hipGetSymbolAddress) with the device current; `stream` must belong to the
 * current device (else MT_ERR_INVALID_ARG). Every call on a device shares that
 * device's array: calls that overlap on one device (other streams, other threads)
 * race and must be serialised by the caller; nothing in the array needs to start at
 * zero (every scratch value is written before it is read). Returns
 * MT_ERR_NOALLOC_LIMIT, before launching anything, when mt_mlp_workspace_bytes(shape)
 * exceeds MT_NOALLOC_SCRATCH_BYTES (e.g. bf16 with M * 4h/tp above ~28M elements);
 * otherwise as mt_mlp_bwd. */
#define MT_NOALLOC_SCRATCH_BYTES (64u << 20)
int mt_mlp_bwd_noalloc(const mt_shape *shape, const void *x, const void *w_fc1, const void *w_fc2,
                       const void *saved, size_t saved_bytes, const void *dy, void *dx_partial, float *dw_fc1,
                       float *db_fc1, float *dw_fc2, void *stream);

/* Attention block alone, the head-parallel counterpart of mt_mlp_* (concept report,
 * section 4.1: heads split over ranks, output projection split by rows):
 *   QKV = u W_qkv^T + b_qkv;  ctx = causal softmax attention over the shard's heads;
 *   o_partial = ctx W_o^T      with u [M, h], W_qkv [3*ht, h], b_qkv [3*ht], W_o [h, ht].
 * No LayerNorm, no b_o, no residual: the sum of o_partial over the tp shards is the
 * unsharded block. MT_BF16 and MT_FP32 only (MT_BF16_QK needs LayerNorm's rounding
 * remainder of u, which a caller-supplied u does not carry: MT_ERR_UNSUPPORTED). */
size_t mt_attn_saved_bytes(const mt_shape *shape);
size_t mt_attn_workspace_bytes(const mt_shape *shape);
int mt_attn_fwd(const mt_shape *shape, const void *u, const void *w_qkv, const void *b_qkv, const void *w_o,
                void *o_partial, void *saved, size_t saved_bytes, void *workspace, size_t workspace_bytes,
                void *stream);
/* Backward given d_o [M, h] (the gradient of the block output): du_partial [M, h]
 * (activation dtype; its sum over shards is the block's input gradient, section 4.2),
 * dw_qkv [3*ht, h], db_qkv [3*ht], dw_o [h, ht] in fp32. u, the weights and `saved` must
 * be those of the forward. */
int mt_attn_bwd(const mt_shape *shape, const void *u, const void *w_qkv, const void *w_o, const void *saved,
                size_t saved_bytes, const void *d_o, void *du_partial, float *dw_qkv, float *db_qkv, float *dw_o,
                void *workspace, size_t workspace_bytes, void *stream);

/* Sequence-parallel share of a layer (concept report, section 4.3: the sequence is split
 * over the same group of devices as the tensor-parallel split, each device keeps one
 * segment and runs LayerNorm locally; section 6.4: activations per device drop to S/tp;
 * section 8(1): the all-reduce split into reduce-scatter and all-gather steps).
 * Rank `shard` owns seq/tp positions of each sequence, rows = micro_batch * seq / tp
 * tokens, stored [rows, h] in (sequence, position) order; seq % tp == 0 is required
 * (MT_ERR_INVALID_ARG). One layer on rank i, the collectives being the caller's:
 *   mt_sp_ln_fwd(x_i)             -> u_i              ; all-gather u   -> U [M, h]
 *   mt_attn_fwd(U)                -> O_i partial      ; reduce-scatter -> O_rs [rows, h]
 *   mt_sp_ln_fwd(x_i, O_rs, b_o)  -> x2_i (fp32), v2_i; all-gather v2  -> V2 [M, h]
 *   mt_mlp_fwd(V2)                -> Y_i partial      ; reduce-scatter -> Y_rs [rows, h]
 *   mt_sp_add_fwd(x2_i, Y_rs, b_fc2) -> out_i
 * and backward with the collectives swapped (all-gather dout, then mt_mlp_bwd,
 * reduce-scatter dV2, mt_sp_ln_bwd for LayerNorm 2, all-gather dX2, mt_attn_bwd,
 * reduce-scatter dU, mt_sp_ln_bwd for LayerNorm 1). The replicated parameters' gradients
 * from the mt_sp_* calls are this rank's partial sums over its rows (the group's
 * all-reduce adds them). MT_BF16 and MT_FP32 only.
 *
 * mt_sp_ln_fwd: resid == NULL: y = LN(x) (bias and x2 unused, may be NULL);
 *   else x2 = x + resid + bias (fp32, unrounded) and y = LN(x2). x, resid, y [rows, h];
 *   gamma, beta, bias [h] in the activation dtype; mean, rstd [rows] fp32 (kept for the
 *   backward). */
int mt_sp_ln_fwd(const mt_shape *shape, const void *x, const void *resid, const void *bias, const void *gamma,
                 const void *beta, float *x2, void *y, float *mean, float *rstd, void *stream);
/* mt_sp_add_fwd: out = x2 + y + bias, x2 fp32 [rows, h], y and out [rows, h], bias [h]. */
int mt_sp_add_fwd(const mt_shape *shape, const float *x2, const void *y, const void *bias, void *out, void *stream);
/* mt_sp_ln_bwd: dx = dres + LN-backward(dy; xin, gamma, mean, rstd) over the rank's rows.
 *   xin: the LayerNorm input (fp32 when xin_f32, e.g. x2; else the activation dtype);
 *   dres: the residual path's gradient (fp32 when dres_f32); dx [rows, h] in the
 *   activation dtype, dx_f32 (may be NULL) an fp32 copy. Column sums over the rows, fp32:
 *   dgamma, dbeta (required); dsum = sum of dx (may be NULL; needs dx_f32, whose values
 *   it sums: MT_ERR_INVALID_ARG otherwise); dres_sum = sum of dres (may be NULL).
 *   LayerNorm 2: xin = x2, dres = dout -> dx = dX2, dsum = db_o, dres_sum = db_fc2.
 *   LayerNorm 1: xin = x, dres = dX2 (fp32) -> dx = dX.
 *   Workspace: mt_sp_ln_workspace_bytes. */
size_t mt_sp_ln_workspace_bytes(const mt_shape *shape);
int mt_sp_ln_bwd(const mt_shape *shape, const void *dy, const void *xin, int xin_f32, const void *gamma,
                 const float *mean, const float *rstd, const void *dres, int dres_f32, void *dx, float *dx_f32,
                 float *dgamma, float *dbeta, float *dsum, float *dres_sum, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Fused AdamW step over n fp32 master parameters, one pass (the oreateai.com
 * Megatron-LM analysis, "In-Depth Analysis of Distributed Training Frameworks for Large
 * Models ... Megatron-LM", section 2.2: the fused optimizer step; section 3.1: beta1 0.9,
 * beta2 0.95). Per parameter, with g = grad_scale * grad, t = step (1-based):
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2
 *   p = p - lr weight_decay p - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * param, exp_avg (m) and exp_avg_sq (v) are updated in place; grad is read; param_bf16
 * (may be NULL) receives bf16(p) rounded to nearest even, the weights the next forward
 * multiplies with. All are device pointers, caller-owned, 16-byte aligned; a layer's
 * tensors can share one flat buffer when each starts at a multiple of 4 elements.
 * Arithmetic in fp32 (bias corrections in double on the host). n == 0 is a no-op.
 * Returns MT_ERR_INVALID_ARG for n < 0, step < 1, a beta outside [0, 1) or a null or
 * misaligned pointer, before launching anything; MT_ERR_HIP if the launch fails. */
int mt_adamw_step(int64_t n, float *param, const float *grad, float *exp_avg, float *exp_avg_sq, void *param_bf16,
                  float lr, float beta1, float beta2, float eps, float weight_decay, float grad_scale, int32_t step,
                  void *stream);

/* Static text of a status code. */
const char *mt_status_string(int status);

/* Per-launch timing (the throughput-breakdown aid). While enabled, each launch whose
 * label contains `label_filter` (NULL or "" = every launch) is bracketed by two HIP
 * events on the call's stream and recorded with its label and algorithmic FLOPs and
 * bytes. The events come from a library-wide pool: while timing is enabled, a call
 * that finds the pool empty creates events (hipEventCreate) inside the call, so a
 * timed call is not a pure launch sequence; mt_timing_reset returns the recorded
 * events to the pool, and they live until the process ends. The flag is atomic and
 * the records and pool are locked, so enabling, resetting and reading are safe from
 * any thread; a call in flight on another thread while the flag flips may or may not
 * be timed. Records persist until mt_timing_reset. mt_timing_get waits for record i's
 * end event and returns its duration in ms. Returns MT_OK or an error status. */
int mt_timing_enable(int enable, const char *label_filter);
int mt_timing_reset(void);
int mt_timing_count(void);
int mt_timing_get(int i, char *label, size_t label_len, float *ms, double *flops, double *bytes);

#ifdef __cplusplus
}
#endif

#endif /* MT_H_ */
