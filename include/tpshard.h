/*
 * tpshard.h — C ABI of libtpshard.so: one rank's share of a tensor-parallel
 * Transformer block on one AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the tensor-parallel split described on the
 * freeguideonline tutorial "Megatron-LM：NVIDIA 的大规模并行训练方案", section
 * "Megatron-LM 核心架构 / 张量并行原理", and on "分布式训练基础：数据并行、模型
 * 并行、流水线并行的基本概念与区别", section 2.2 ("核心原理"):
 *   - a column-parallel linear Y = XA with A = [A_1, ..., A_p] split by columns:
 *     rank i computes Y_i = X A_i from the replicated input X;
 *   - a row-parallel linear with A split by rows and X by columns: rank i
 *     computes the partial X_i A_i that an AllReduce would sum;
 *   - in a Transformer, QKV and the MLP's first layer are column-parallel, the
 *     attention output projection and the MLP's second layer row-parallel, and
 *     (tutorial, section "融合优化技术") the bias add and GeLU are fused into
 *     the producing kernel instead of making extra memory round-trips.
 * The backward entry points are the chain rule of these products (the pages
 * say only that tensor parallelism communicates in every layer's forward and
 * backward; the library stops at the per-rank partials, before any sum).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  All matrices are dense, row-major, leading dimension = number of
 *   columns.  Activations are [T x features] with T = tokens (micro-batch x
 *   sequence flattened).  Weights are [in x out] (Y = X W).  Rank i owns the
 *   contiguous column block i (column-parallel) or row block i (row-parallel);
 *   callers pass the shard itself, already sliced and contiguous.
 * Dimensions.  K = full in-features, N = full out-features, p = tp_size >= 1.
 *   The shard width is N/p (column) or K/p (row) and must be an integer
 *   (TP_ERR_TP_DIVISIBILITY).  T >= 1 is arbitrary; every feature dimension
 *   (K, N, and their shard widths) must be a positive multiple of 8
 *   (TP_ERR_ALIGNMENT) and at most 2^21 (TP_ERR_DIM); T must be <= 2^30
 *   (TP_ERR_DIM).
 * Dtypes.  dtype = TP_BF16: activations, weights, biases and activation
 *   outputs are bfloat16; products accumulate in fp32 on the matrix cores
 *   and are rounded to nearest-even on store.  dtype = TP_FP32: everything is
 *   fp32 with fp32 arithmetic (a check path).  dtype = TP_FP16: as TP_BF16 with
 *   IEEE half storage and the fp16 matrix-core instruction -- the fp16 mixed-
 *   precision path, used with dynamic loss scaling (tp_unscale_check_finite)
 *   because half's range is narrow ([TUT] "最佳实践与调优建议" and "常见问题").
 *   Parameter gradients (dW, db) are always fp32, for every dtype.  Core
 *   attention takes TP_BF16 only.
 * Pointers.  Device pointers (hipMalloc / torch CUDA tensors), 16-byte aligned
 *   (TP_ERR_ALIGNMENT).  Required pointers must be non-NULL (TP_ERR_NULLPTR).
 *   No output may overlap any input or another output (TP_ERR_ALIAS).
 * Ownership.  The caller owns every buffer.  The library never allocates,
 *   frees or retains device memory; scratch comes only from `workspace`,
 *   whose size is given by tp_workspace_size().
 * Streams.  `stream` is a hipStream_t (NULL = the legacy default stream).
 *   Every call only enqueues work on it and returns; the caller synchronises.
 *   Calls that share a workspace must be ordered on one stream.
 * Errors.  Returns TP_OK (0) or a negative status (tp_status_string gives the
 *   text).  All argument checks run before anything is enqueued: on a
 *   validation error nothing is launched and no output is touched.  A failed
 *   launch returns TP_ERR_HIP.  No C++ exception or abort crosses the ABI.
 * Determinism.  No floating-point atomics: equal inputs give bitwise equal
 *   outputs on every run.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TP_BF16 = 0, TP_FP32 = 1, TP_FP16 = 2 } tp_dtype;
typedef enum { TP_ACT_NONE = 0, TP_ACT_GELU = 1 } tp_act;

enum {
  TP_OK = 0,
  TP_ERR_NULLPTR = -1,          /* a required pointer is NULL */
  TP_ERR_DIM = -2,              /* a dimension is < 1 or too large (T > 2^30, feature > 2^21) */
  TP_ERR_TP_DIVISIBILITY = -3,  /* tp_size < 1 or the sharded dimension not divisible by it */
  TP_ERR_ALIGNMENT = -4,        /* pointer not 16-byte aligned or feature dim not a multiple of 8 */
  TP_ERR_DTYPE = -5,            /* unknown dtype or activation code */
  TP_ERR_ALIAS = -6,            /* an output overlaps an input or another output */
  TP_ERR_WORKSPACE = -7,        /* workspace NULL or smaller than tp_workspace_size() */
  TP_ERR_HIP = -8,              /* a HIP runtime call or kernel launch failed */
  TP_ERR_ARG = -9,              /* other invalid argument (flag value, unexpected pointer) */
  TP_ERR_SCRATCH = -10          /* more scratch needed than tp_noalloc_scratch_bytes() (the
                                   allocation-free entry point only) */
};

/* Operation codes for tp_workspace_size(). */
enum {
  TP_OP_COLUMN_LINEAR_BWD = 1,
  TP_OP_ROW_LINEAR_BWD = 2,
  TP_OP_MLP_SHARD_BWD = 3,
  TP_OP_BIAS_GRAD = 4,
  TP_OP_ATTENTION_BWD = 5,
  TP_OP_MLP_SHARD_BWD_RECOMPUTE = 6,
  TP_OP_LAYERNORM_BWD = 7,
  TP_OP_BIAS_DROPOUT_ADD_BWD = 8
};

/*
 * Column-parallel linear, forward (tutorial "张量并行原理": Y_i = X A_i).
 *   X   [T x K]     replicated input
 *   W_i [K x N/p]   this rank's column block of W
 *   b_i [N/p]       this rank's bias block, or NULL
 *   act TP_ACT_NONE: Y_i = X W_i + b_i; Z_i must be NULL.
 *       TP_ACT_GELU: Z_i = X W_i + b_i (stored only if Z_i != NULL) and
 *                    Y_i = GeLU(Z_i) = Z_i * Phi(Z_i) (exact erf form), both
 *                    computed from the fp32 accumulators in one kernel.
 *   Y_i, Z_i [T x N/p], dtype.
 */
int tp_column_linear(const void* X, const void* W_i, const void* b_i, void* Y_i, void* Z_i,
                     int64_t T, int64_t K, int64_t N, int32_t tp_size, int32_t act, int32_t dtype,
                     void* stream);

/*
 * Row-parallel linear, forward (tutorial "张量并行原理": A split by rows, X by
 * columns; the partials are summed by an AllReduce outside this library).
 *   X_i [T x K/p]   this rank's column block of the input
 *   W_i [K/p x N]   this rank's row block of W
 *   b   [N]         output bias or NULL; pass it on exactly one rank, since the
 *                   partials are summed afterwards
 *   Y_i [T x N]     partial output X_i W_i (+ b), dtype
 */
int tp_row_linear(const void* X_i, const void* W_i, const void* b, void* Y_i,
                  int64_t T, int64_t K, int64_t N, int32_t tp_size, int32_t dtype, void* stream);

/*
 * MLP shard, forward: the first layer column-parallel, then the fused bias +
 * GeLU, then the second layer row-parallel (tutorial "张量并行原理", last
 * paragraph, and "融合优化技术").  With f = F/p:
 *   X    [T x h]  replicated input        A_i [h x f]   B_i [f x h]
 *   b1_i [f] or NULL
 *   Z_i  [T x f]  = X A_i + b1_i, saved for the backward; NULL = inference
 *   H_i  [T x f]  = GeLU(Z_i)  (written once, already activated)
 *   Y_i  [T x h]  = H_i B_i, the rank's partial (no output bias; it is added
 *                   once after the row-parallel sum)
 */
int tp_mlp_shard_fwd(const void* X, const void* A_i, const void* b1_i, const void* B_i,
                     void* Z_i, void* H_i, void* Y_i,
                     int64_t T, int64_t h, int64_t F, int32_t tp_size, int32_t dtype, void* stream);

/*
 * MLP shard, backward.  Inputs are the forward's X, A_i, B_i and the saved
 * Z_i, H_i, plus dY [T x h] = dL/dY (gradient of the summed output).
 *   dB_i  [f x h] fp32 = H_i^T dY
 *   dZ            = (dY B_i^T) * GeLU'(Z_i), GeLU'(z) = Phi(z) + z phi(z)
 *                   (kept in the workspace, dtype)
 *   db1_i [f]     fp32 = sum over tokens of dZ, or NULL to skip
 *   dA_i  [h x f] fp32 = X^T dZ
 *   dX_i  [T x h] dtype = dZ A_i^T (this rank's partial of dX)
 *   db2   [h]     fp32 = sum over tokens of dY (gradient of the row-parallel
 *                   output bias; compute it on one rank), or NULL to skip
 *   accumulate 0: overwrite dA_i, dB_i, db1_i, db2; 1: add to them.
 *   workspace: >= tp_workspace_size(TP_OP_MLP_SHARD_BWD, T, h, F, p, dtype) bytes:
 *   dZ, the bias-gradient partial rows, and (16-bit, where a weight gradient's
 *   tiles would fill at most half of the CUs and T is at least 2048) the fp32
 *   partial of that GEMM's K split: twice the workgroups each take half of the
 *   tokens, and a second pass adds the second half to the first in a fixed
 *   order (with accumulate: (old + first half) + second half).
 */
int tp_mlp_shard_bwd(const void* X, const void* A_i, const void* B_i, const void* Z_i,
                     const void* H_i, const void* dY, void* dX_i, float* dA_i, float* db1_i,
                     float* dB_i, float* db2, void* workspace, size_t workspace_bytes,
                     int32_t accumulate, int64_t T, int64_t h, int64_t F, int32_t tp_size,
                     int32_t dtype, void* stream);

/*
 * MLP shard backward that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory or hand out scratch: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, outputs, kernels and results (bitwise) as tp_mlp_shard_bwd,
 * without workspace / workspace_bytes: the scratch (dZ, the bias-gradient
 * partials, a K split's partial) lives in a static device array of tp_noalloc_scratch_bytes()
 * (96 MiB) that the library holds on each GPU it runs on until the process
 * ends.  A problem whose scratch, tp_workspace_size(TP_OP_MLP_SHARD_BWD, ...),
 * exceeds that size is rejected with TP_ERR_SCRATCH before anything is
 * enqueued (the 175B TP=8 shard needs 26 MiB, the 1.3B TP=1 MLP 64.3 MiB in
 * 16-bit storage).  No hipMalloc, hipFree or allocating library routine is
 * called; the first call on a GPU looks the array's device address up once.
 * Every call on a GPU uses that GPU's one array: calls that overlap in time on
 * one GPU (different streams, or different host threads without ordering)
 * race on it and must not be issued.  The array keeps the last call's
 * contents; nothing in it needs to start at zero.
 */
int tp_mlp_shard_bwd_noalloc(const void* X, const void* A_i, const void* B_i, const void* Z_i,
                             const void* H_i, const void* dY, void* dX_i, float* dA_i, float* db1_i,
                             float* dB_i, float* db2, int32_t accumulate, int64_t T, int64_t h, int64_t F,
                             int32_t tp_size, int32_t dtype, void* stream);

/* Bytes of the static scratch array of tp_mlp_shard_bwd_noalloc. */
size_t tp_noalloc_scratch_bytes(void);

/*
 * MLP shard backward with selective activation recompute ([TUT] "融合优化技术"
 * and "高级特性 / 选择性激活重计算": keep fewer activations from the forward
 * and recompute the rest in the backward, trading compute for memory).
 * Same outputs and conventions as tp_mlp_shard_bwd; the forward's saved
 * activations are replaced by:
 *   Z_i non-NULL: only the pre-activation was kept; H_i = GeLU(Z_i) is
 *                 recomputed in the epilogue of the dZ GEMM, which reads Z_i
 *                 for GeLU' anyway (H_i need not be kept; no extra pass);
 *   Z_i NULL:     nothing was kept; Z_i and H_i are recomputed by the
 *                 forward's fused fc1 GEMM (X A_i + b1_i, then GeLU), which
 *                 needs b1_i (NULL = no bias) -- bitwise the forward's values.
 * The recomputed tensors live in the workspace: >= tp_workspace_size(
 * TP_OP_MLP_SHARD_BWD_RECOMPUTE, T, h, F, p, dtype) bytes.
 */
int tp_mlp_shard_bwd_recompute(const void* X, const void* A_i, const void* b1_i, const void* B_i,
                               const void* Z_i, const void* dY, void* dX_i, float* dA_i, float* db1_i,
                               float* dB_i, float* db2, void* workspace, size_t workspace_bytes,
                               int32_t accumulate, int64_t T, int64_t h, int64_t F, int32_t tp_size,
                               int32_t dtype, void* stream);

/*
 * Column-parallel linear, backward (no activation; for the GeLU layer use
 * tp_mlp_shard_bwd).  X [T x K], W_i [K x N/p], dY_i [T x N/p]:
 *   dX_partial [T x K]   dtype = dY_i W_i^T (summed over ranks outside)
 *   dW_i       [K x N/p] fp32  = X^T dY_i
 *   db_i       [N/p]     fp32  = sum over tokens of dY_i, or NULL
 *   accumulate as in tp_mlp_shard_bwd.  workspace: TP_OP_COLUMN_LINEAR_BWD bytes,
 *   required with db_i.  A workspace of that size also lets a small dW_i (tiles
 *   filling at most half of the CUs, T >= 2048) split its contraction as in
 *   tp_mlp_shard_bwd; with none (db_i NULL) dW_i is computed unsplit.
 */
int tp_column_linear_bwd(const void* X, const void* W_i, const void* dY_i, void* dX_partial,
                         float* dW_i, float* db_i, void* workspace, size_t workspace_bytes,
                         int32_t accumulate, int64_t T, int64_t K, int64_t N, int32_t tp_size,
                         int32_t dtype, void* stream);

/*
 * Row-parallel linear, backward.  X_i [T x K/p], W_i [K/p x N], dY [T x N]:
 *   dX_i [T x K/p] dtype = dY W_i^T (exact gradient of this rank's input block)
 *   dW_i [K/p x N] fp32  = X_i^T dY
 *   db   [N]       fp32  = sum over tokens of dY, or NULL (one rank only)
 *   accumulate as above.  workspace: TP_OP_ROW_LINEAR_BWD bytes, required
 *   with db; it also lets a small dW_i split its contraction, as above.
 */
int tp_row_linear_bwd(const void* X_i, const void* W_i, const void* dY, void* dX_i,
                      float* dW_i, float* db, void* workspace, size_t workspace_bytes,
                      int32_t accumulate, int64_t T, int64_t K, int64_t N, int32_t tp_size,
                      int32_t dtype, void* stream);

/*
 * Bias gradient alone: db [N] fp32 (=, or += with accumulate) sum over the T
 * rows of dY [T x N] (dtype).  workspace: TP_OP_BIAS_GRAD with d_in = N.
 */
int tp_bias_grad(const void* dY, float* db, void* workspace, size_t workspace_bytes,
                 int32_t accumulate, int64_t T, int64_t N, int32_t dtype, void* stream);

/*
 * The bias + GeLU step as a separate elementwise pass (the unfused form that
 * the fused epilogue replaces; kept for measurement):
 *   H [T x N] = GeLU(Z + b), Z [T x N], b [N] (or NULL), dtype.
 */
int tp_bias_gelu(const void* Z, const void* b, void* H, int64_t T, int64_t N, int32_t dtype,
                 void* stream);

/*
 * Core attention on the rank's local heads.  [TUT] "Megatron-LM 核心架构 /
 * 张量并行原理": with the Q, K, V projections column-parallel and the output
 * projection row-parallel, each rank owns whole heads and runs their attention
 * locally between the two shards; [INTRO] "课程导入" 1.3.1: multi-head
 * self-attention; [TUT] "最佳实践与调优建议": an IO-aware exact attention kernel
 * (the score matrix never reaches HBM).
 *
 *   Hl = heads / tp_size local heads of width head_dim (64 or 128);
 *   QKV_i [T x 3*Hl*head_dim] bf16: columns [Q | K | V], each block head-major
 *         ([head][head_dim]) -- the QKV column shard's output;
 *   T = B * seq tokens: B sequences of length seq packed back to back;
 *   O_i [T x Hl*head_dim] bf16, head-major -- the out-projection row shard's input;
 *   per head and sequence O = softmax(Q K^T / sqrt(head_dim) + M) V, M the causal
 *   mask (key > query excluded) when causal = 1, none when causal = 0; scores and
 *   softmax in fp32; no dropout;
 *   lse [Hl x T] fp32 (nullable, e.g. for inference): natural-log log-sum-exp of
 *   each query's scaled scores over its allowed keys (what the backward reads).
 * dtype must be TP_BF16 (TP_ERR_DTYPE for TP_FP32 and TP_FP16).  Errors: head_dim not 64/128,
 * T not a multiple of seq, or 3*Hl*head_dim > 2^21 -> TP_ERR_DIM; heads not
 * divisible by tp_size -> TP_ERR_TP_DIVISIBILITY; causal not 0/1 -> TP_ERR_ARG;
 * outputs overlapping the input or each other -> TP_ERR_ALIAS.
 */
int tp_attention_fwd(const void* QKV_i, void* O_i, float* lse, int64_t T, int64_t seq, int64_t heads,
                     int64_t head_dim, int32_t tp_size, int32_t causal, int32_t dtype, void* stream);

/*
 * Backward of tp_attention_fwd (the chain rule of the same definition; the
 * pages give no backward formulas).  Inputs: QKV_i, O_i and lse as written by
 * the forward with the same arguments, dO_i [T x Hl*head_dim] bf16.  Output:
 * dQKV_i [T x 3*Hl*head_dim] bf16 in the same [Q | K | V] layout, which is
 * the dY_i the QKV column shard's backward (tp_column_linear_bwd) takes.
 * Computed without atomics (bitwise reproducible).  workspace: >=
 * tp_workspace_size(TP_OP_ATTENTION_BWD, T, heads, head_dim, tp_size, TP_BF16)
 * bytes (TP_ERR_WORKSPACE).  Errors as tp_attention_fwd; lse is required here.
 */
int tp_attention_bwd(const void* QKV_i, const void* O_i, const float* lse, const void* dO_i, void* dQKV_i,
                     void* workspace, size_t workspace_bytes, int64_t T, int64_t seq, int64_t heads,
                     int64_t head_dim, int32_t tp_size, int32_t causal, int32_t dtype, void* stream);

/*
 * Sequence-parallel edge steps on the rank's rows ([TUT] "序列并行": on top of
 * tensor parallelism, LayerNorm and Dropout are split along the sequence
 * dimension; [INTRO] "课程导入" 1.4.2: sequence parallelism cuts the sequence
 * and communicates at LayerNorm / Dropout).  rows = the rank's tokens, h = the
 * hidden size (a multiple of 8, <= 2^21); dtype bf16 or fp32 as elsewhere;
 * statistics and parameter gradients fp32.
 *
 * LayerNorm forward: Y = (X - mean) / sqrt(var + eps) * gamma + beta per row
 * (var the biased variance over h), X, Y [rows x h], gamma [h], beta [h] or
 * NULL; mean, rstd [rows] fp32 = the row mean and 1/sqrt(var + eps) (both
 * NULL for inference, else both given: TP_ERR_ARG).  eps >= 0 (TP_ERR_ARG).
 */
int tp_layernorm_fwd(const void* X, const void* gamma, const void* beta, void* Y, float* mean, float* rstd,
                     int64_t rows, int64_t h, float eps, int32_t dtype, void* stream);
/*
 * LayerNorm backward (chain rule of the forward): from X, gamma and the
 * forward's mean / rstd, and dY [rows x h]:
 *   dX [rows x h] dtype = rstd * (g - mean_h(g) - xhat * mean_h(g * xhat)),
 *                 g = dY * gamma, xhat = (X - mean) * rstd;
 *   dgamma [h] fp32 = sum over rows of dY * xhat;  dbeta [h] fp32 = sum of dY
 *   (NULL to skip).  accumulate 0/1 as for the MLP.  Deterministic.
 * workspace: >= tp_workspace_size(TP_OP_LAYERNORM_BWD, rows, h, 0, 1, dtype).
 */
int tp_layernorm_bwd(const void* X, const void* gamma, const float* mean, const float* rstd, const void* dY,
                     void* dX, float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes,
                     int32_t accumulate, int64_t rows, int64_t h, int32_t dtype, void* stream);
/*
 * Bias + dropout + residual add after the row-parallel output (one fused pass,
 * [TUT] "融合优化技术"):  out = residual + keep * (Y + b) / (1 - p_drop), with
 * Y, residual, out [rows x h], b [h] or NULL, 0 <= p_drop < 1 (TP_ERR_ARG).
 * keep: element e (row-major index) is kept when word (offset + e) mod 4 of
 * Philox4x32-10 (Salmon et al., SC'11) with counter ((offset + e) / 4, 0, 0)
 * -- 64-bit block number in the first two words -- and key (seed low 32 bits,
 * seed high 32 bits) is below floor((1 - p_drop) * 2^32).  offset is an
 * element counter (a multiple of 8, TP_ERR_ARG), so callers give each layer
 * and rank a disjoint range; the backward regenerates the same mask.
 */
int tp_bias_dropout_add_fwd(const void* Y, const void* b, const void* residual, void* out, int64_t rows, int64_t h,
                            double p_drop, uint64_t seed, uint64_t offset, int32_t dtype, void* stream);
/*
 * Its backward: dY [rows x h] dtype = keep * dOut / (1 - p_drop) (same mask);
 * db [h] fp32 = sum over rows of dY (NULL to skip; then no workspace is
 * needed), accumulate 0/1; the residual's gradient is dOut itself.
 * workspace: >= tp_workspace_size(TP_OP_BIAS_DROPOUT_ADD_BWD, rows, h, 0, 1, dtype).
 */
int tp_bias_dropout_add_bwd(const void* dOut, void* dY, float* db, void* workspace, size_t workspace_bytes,
                            int32_t accumulate, int64_t rows, int64_t h, double p_drop, uint64_t seed,
                            uint64_t offset, int32_t dtype, void* stream);

/*
 * Loss-scaling hook of the fp16 path ([TUT] "常见问题": a loss that turns NaN
 * under fp16 calls for dynamic loss scaling; [INTRO] 1.4.1: fp32 master
 * weights).  For an fp32 gradient buffer grads[n] (device, 16-byte aligned):
 * grads *= inv_scale in place, and *found_nonfinite (device int32, 4-byte
 * aligned) is set to 1 if any element is inf or NaN -- it is never cleared,
 * so one flag can collect several buffers; the caller zeroes it before the
 * step and skips the optimizer step (and lowers the scale) when it is set.
 * inv_scale > 0 and finite (TP_ERR_ARG); 1 <= n <= 2^36 (TP_ERR_DIM).
 */
int tp_unscale_check_finite(float* grads, int64_t n, float inv_scale, int32_t* found_nonfinite, void* stream);

/*
 * Workspace bytes needed by `op` (TP_OP_*).  Arguments are those of the
 * matching call: T, d_in, d_out = (T, K, N) for the linears, (T, h, F) for the
 * MLP and its recompute form, (T, N, unused) for the bias gradient, (T, heads, head_dim) for the
 * attention backward (dtype TP_BF16), (rows, h, unused) for the LayerNorm and
 * bias-dropout-add backwards.  Returns 0 for invalid arguments.  In the linear
 * and MLP backwards it holds the bias-gradient partials: with 16-bit storage
 * most weight-gradient tile shapes add the columns of dY while dY passes
 * through the GEMM and leave one fp32 row per row of tiles; otherwise a
 * column-sum pass over dY leaves its own partial rows.  The MLP backward also
 * keeps dZ there (and the recompute form H and Z).
 */
size_t tp_workspace_size(int32_t op, int64_t T, int64_t d_in, int64_t d_out, int32_t tp_size,
                         int32_t dtype);

/* Static, NUL-terminated text for a status code. */
const char* tp_status_string(int status);

/*
 * Kernel timing trace (measurement aid).  While a trace is open, every kernel
 * the library launches is bracketed by a pair of hipEvents recorded on the
 * stream it is launched on, together with its algorithmic FLOP and HBM byte
 * counts.  tp_trace_start(max_launches) opens a trace with room for that many
 * launches (events are created here; launches past the limit are not
 * recorded); tp_trace_stop() waits for the recorded events and aggregates
 * them per kernel name.  Not thread-safe: one host thread drives a trace.
 */
int tp_trace_start(int32_t max_launches);
int tp_trace_stop(void);
/* Number of distinct kernels in the last stopped trace. */
int tp_trace_num_kernels(void);
/* Kernel `idx` of the last stopped trace: name (truncated to name_len-1),
 * number of launches, summed duration (ms), summed algorithmic FLOP and bytes. */
int tp_trace_kernel(int32_t idx, char* name, size_t name_len, int64_t* launches,
                    double* total_ms, double* flops, double* bytes);

/*
 * Matrix-core probe (measurement only; no layer arithmetic).  Launches
 * `blocks` workgroups of 4 waves; every wave issues 16 * `iters` bf16 MFMAs
 * (32x32x16, fp32 accumulate, 32768 FLOP each) on register operands with
 * random bits and no memory traffic, so the run shows what the matrix cores
 * sustain under the board's power limit.  Outputs (device memory, caller
 * owned): sink[blocks * 256] floats (one accumulator sum per thread, written
 * only so the work is kept); ticks[2 * blocks] as unsigned 64-bit integers,
 * per workgroup: shader-clock cycles, then constant-rate-clock ticks (rate
 * from tp_wall_clock_rate_khz) spent in its MFMA loop.  Asynchronous on
 * `stream`.  Limits: 1 <= blocks <= 65536, 1 <= iters <= 2^24, else
 * TP_ERR_ARG; null outputs TP_ERR_NULLPTR; ticks not 8-byte aligned
 * TP_ERR_ALIGNMENT; launch failure TP_ERR_HIP.
 */
int tp_mfma_probe(int32_t blocks, int32_t iters, float* sink, unsigned long long* ticks, void* stream);
/* Rate of the constant-rate clock read by tp_mfma_probe (kHz) on the current
 * device, written to *khz.  TP_ERR_NULLPTR for a null khz, TP_ERR_HIP when
 * the runtime cannot report it. */
int tp_wall_clock_rate_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
