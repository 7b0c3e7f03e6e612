// Matrix-core throughput probe (measurement only, not part of any layer's
// arithmetic).  Every wave streams the same bf16 MFMA the GEMMs use
// (32x32x16, fp32 accumulate) from registers, with no memory traffic, on
// high-entropy operands that change from one instruction to the next, so the
// multipliers toggle about as much as they do in a GEMM on random data.  Each
// workgroup also records how many shader-clock and constant-rate-clock ticks
// its loop took, from which the caller reads the clock the chip sustained.
// Together they give the throughput the matrix cores reach under the board's
// power limit, the ceiling a GEMM's rate is best compared against beside the
// datasheet peak.
#include "side.h"

namespace tps {
namespace {

constexpr int PROBE_THREADS = 256;  // 4 waves

// 32-bit integer finaliser (two multiply-xorshift rounds), used only to give
// the operands well-mixed bits.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ bf16 rand_bf16(uint32_t key) {
  // uniform in [-2, 2): random sign, exponent and full 7-bit mantissa
  return (bf16)((float)((int)(mix32(key) & 0xffffu) - 32768) * (1.0f / 16384.0f));
}

__global__ void __launch_bounds__(PROBE_THREADS) mfma_probe_kernel(int iters, float* sink,
                                                                   unsigned long long* ticks) {
  const uint32_t tid = blockIdx.x * PROBE_THREADS + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[q][e] = rand_bf16(tid * 64u + q * 8u + e);
      b[q][e] = rand_bf16(tid * 64u + q * 8u + e + 0x9e3779b9u);
    }
  f32x16 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x16{};
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
    // 16 MFMAs: four independent accumulator chains, each pairing its A
    // operand with a rotating B operand
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q], b[(q + r) & 3], acc[q], 0, 0, 0);
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[q][e];
  sink[tid] = s;
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = c1 - c0;
    ticks[2 * blockIdx.x + 1] = w1 - w0;
  }
}

}  // namespace

hipError_t mfma_probe(int blocks, int iters, float* sink, unsigned long long* ticks, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(PROBE_THREADS), 0, s, iters, sink, ticks);
  return hipGetLastError();
}

}  // namespace tps
