// Internal declarations shared by the kernels and the C-ABI layer of
// libtpshard.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace tps {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// Epilogue applied to the fp32 accumulators of a GEMM tile.
enum Epi : int {
  EPI_STORE = 0,      // C (dtype) = acc (+ bias[n])
  EPI_BIAS_GELU = 1,  // z = acc (+ bias[n]); C2 (dtype, optional) = z; C (dtype) = GeLU(z)
  EPI_DGELU = 2,      // C (dtype) = acc * GeLU'(aux[m, n])
  EPI_F32 = 3         // C (fp32) = acc, or C += acc when accumulate
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
  void* C2;           // second output (pre-activation for EPI_BIAS_GELU), nullable
  int64_t ldc2;
  const void* bias;   // [N], dtype of the path, nullable
  const void* aux;    // [M x N] read by EPI_DGELU
  int64_t ldaux;
  int accumulate;     // EPI_F32 only
  int group_m;        // tile rows per group in the tile order (set by the launcher)
};

// Kernel launch record for the optional event trace.
struct LaunchInfo {
  const char* name;
  double flops;
  double bytes;
};

// Trace hooks (api.cpp). begin/end bracket a launch on `stream`.
void trace_begin(hipStream_t stream);
void trace_end(hipStream_t stream, const LaunchInfo& info);

// GEMM launchers (gemm_bf16.hip / gemm_f32.hip). Return hipSuccess or the
// launch error.  a_kcontig / b_kcontig select the operand layouts.
hipError_t gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s);
hipError_t gemm_f32(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s);

// Column sum over rows (elementwise.hip): out[n] (+)= sum_t in[t, n].
// Uses `chunks * N` floats of workspace.
int colsum_chunks(int64_t T, int64_t N);
hipError_t colsum(const void* in, bool in_bf16, float* out, float* ws, int accumulate,
                  int64_t T, int64_t N, hipStream_t s);

// H = GeLU(Z + b) elementwise (elementwise.hip).
hipError_t bias_gelu(const void* Z, const void* b, void* H, bool is_bf16, int64_t T, int64_t N,
                     hipStream_t s);

// Register-only MFMA throughput probe (probe.hip).
hipError_t mfma_probe(int blocks, int iters, float* sink, unsigned long long* ticks, hipStream_t s);

}  // namespace tps
