// GEMM launch arguments and launchers (gemm_bf16.hip, gemm_f32.hip).
#pragma once

#include "common.h"

namespace tps {

// Epilogue applied to the fp32 accumulators of a GEMM tile.
enum Epi : int {
  EPI_STORE = 0,      // C (dtype) = acc (+ bias[n])
  EPI_BIAS_GELU = 1,  // z = acc (+ bias[n]); C2 (dtype, optional) = z; C (dtype) = GeLU(z)
  EPI_DGELU = 2,      // C (dtype) = acc * GeLU'(aux[m, n])
  EPI_F32 = 3,        // C (fp32) = acc, or C += acc when accumulate
  EPI_DGELU_H = 4     // as EPI_DGELU, and C2 (dtype) = GeLU(aux[m, n]) from the same erf evaluation
};

// One C = op(A)[M x K] * op(B)[K x N] launch plus its epilogue operands.
// A is [M x K] row-major when a_kcontig, else [K x M] row-major (A^T stored);
// B is [N x K] row-major when b_kcontig, else [K x N] row-major.
struct GemmArgs {
  const void* A;
  const void* B;
  int64_t lda, ldb;
  int M, N, K;
  void* C;            // main output
  int64_t ldc;
  void* C2;           // second output: the pre-activation for EPI_BIAS_GELU (nullable), GeLU(aux) for EPI_DGELU_H
  int64_t ldc2;
  const void* bias;   // [N], dtype of the path, nullable
  const void* aux;    // [M x N] read by EPI_DGELU
  int64_t ldaux;
  int accumulate;     // EPI_F32 only
  // 16-bit EPI_F32 with B stored [K x N] only, nullable: partial column sums of
  // B over K, gemm16_colsum_rows(M, N, K, kpart != nullptr) rows of N floats (row r = the sum over
  // a subset of K, the rows together cover K once).  Adding the rows gives the
  // bias gradient that goes with a weight gradient dW = X^T dY (db = sum_t dY).
  float* colsum;
  // 16-bit EPI_F32 with both operands stored [K x *] only, nullable: room for an
  // M x N fp32 partial.  When gemm16_ksplit(M, N, K), the launch splits K in two
  // halves over twice the workgroups; the first half's tiles write C as usual,
  // the second's write their partial here, and a second pass adds it to C.
  float* kpart;
  int group_m;        // tile rows per group in the tile order (set by the launcher)
};

// GEMM launchers (gemm_bf16.hip / gemm_f32.hip). Return hipSuccess or the
// launch error.  a_kcontig / b_kcontig select the operand layouts.
hipError_t gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s);
hipError_t gemm_f16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s);
hipError_t gemm_f32(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s);

// Two independent products in one launch: g1 a data gradient (both operands
// K-contiguous, epi1 EPI_STORE or EPI_DGELU), g2 a weight gradient (both
// operands [K x *], EPI_F32, its column sums optional, never K-split).
// Returns hipErrorNotSupported, having launched nothing, unless
// gemm16_pairs(g1.M, g1.N, g1.K, g2.M, g2.N, g2.K, ...) holds; the results are
// those of the two launches made one after the other.
hipError_t gemm_bf16_pair(const GemmArgs& g1, Epi epi1, const GemmArgs& g2, hipStream_t s);
hipError_t gemm_f16_pair(const GemmArgs& g1, Epi epi1, const GemmArgs& g2, hipStream_t s);
// Whether the pair runs as one launch (split2: g2.kpart is set).
bool gemm16_pairs(int M1, int N1, int K1, int M2, int N2, int K2, bool split2);

// Work-items of the launch gemm_bf16 / gemm_f16 (resp. gemm_f32) makes for an
// M x N product: every launch must stay within the 32-bit dispatch size.
int64_t gemm16_work_items(int64_t M, int64_t N);
int64_t gemm_f32_work_items(int64_t M, int64_t N);

// Rows of GemmArgs::colsum written by the 16-bit GEMM for an M x N product with
// contraction K, with (kpart) or without room for a K split's partial.
int gemm16_colsum_rows(int M, int N, int K, bool kpart);

// Whether the 16-bit weight-gradient GEMM (EPI_F32, both operands [K x *])
// splits K in two for an M x N product with contraction K, given kpart: when
// its tiles would fill at most half of the CUs and K >= 2048 (each half keeps
// at least 32 K steps).
bool gemm16_ksplit(int M, int N, int K);

}  // namespace tps
