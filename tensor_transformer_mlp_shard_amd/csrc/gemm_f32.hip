// fp32 GEMM with the same epilogues as the bf16 path: the fp32 check path.
//
// Plain LDS-tiled FMA kernel (64 x 64 output tile, K step 16, 256 threads with
// 4 x 4 outputs each).  It exists to run the whole shard in true fp32
// arithmetic, not for speed; the bf16 matrix-core kernel is the product path.
#include "gemm.h"

namespace tps {
namespace {

constexpr int TB = 64;  // output tile edge
constexpr int TK = 16;  // K step

__device__ __forceinline__ float gelu32(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.7071067811865475f));
}

__device__ __forceinline__ float gelu_grad32(float z) {
  const float cdf = 0.5f * (1.0f + erff(z * 0.7071067811865475f));
  const float pdf = 0.3989422804014327f * expf(-0.5f * z * z);
  return cdf + z * pdf;
}

template <bool AK, bool BKC, int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[TK][TB + 1];  // [k][m]
  __shared__ float Bs[TK][TB + 1];  // [k][n]
  const float* __restrict__ A = (const float*)g.A;
  const float* __restrict__ B = (const float*)g.B;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  // one flat grid over the tiles (a second grid dimension would cap M at 65536 tiles)
  const int tiles_n = (g.N + TB - 1) / TB;
  const int m0 = (int)(blockIdx.x / tiles_n) * TB, n0 = (int)(blockIdx.x % tiles_n) * TB;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < g.K; k0 += TK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;
      int m, k;
      if (AK) { m = idx / TK; k = idx % TK; } else { k = idx / TB; m = idx % TB; }
      const int gm = m0 + m, gk = k0 + k;
      float v = 0.0f;
      if (gm < g.M && gk < g.K) v = AK ? A[(int64_t)gm * g.lda + gk] : A[(int64_t)gk * g.lda + gm];
      As[k][m] = v;
      int n;
      if (BKC) { n = idx / TK; k = idx % TK; } else { k = idx / TB; n = idx % TB; }
      const int gn = n0 + n, gk2 = k0 + k;
      float w = 0.0f;
      if (gn < g.N && gk2 < g.K) w = BKC ? B[(int64_t)gn * g.ldb + gk2] : B[(int64_t)gk2 * g.ldb + gn];
      Bs[k][n] = w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= g.N) continue;
      float v = acc[i][j];
      if (EPI == EPI_F32) {
        float* c = (float*)g.C + (int64_t)m * g.ldc + n;
        *c = g.accumulate ? *c + v : v;
        continue;
      }
      if ((EPI == EPI_STORE || EPI == EPI_BIAS_GELU) && g.bias != nullptr) v += ((const float*)g.bias)[n];
      if (EPI == EPI_BIAS_GELU) {
        if (g.C2 != nullptr) ((float*)g.C2)[(int64_t)m * g.ldc2 + n] = v;
        v = gelu32(v);
      }
      if (EPI == EPI_DGELU || EPI == EPI_DGELU_H) {
        const float z = ((const float*)g.aux)[(int64_t)m * g.ldaux + n];
        v *= gelu_grad32(z);
        if (EPI == EPI_DGELU_H) ((float*)g.C2)[(int64_t)m * g.ldc2 + n] = gelu32(z);
      }
      ((float*)g.C)[(int64_t)m * g.ldc + n] = v;
    }
  }
}

template <bool AK, bool BKC, int EPI>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  const dim3 grid((unsigned)(((int64_t)g.N + TB - 1) / TB * (((int64_t)g.M + TB - 1) / TB)));
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, EPI>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int64_t gemm_f32_work_items(int64_t M, int64_t N) { return (M + TB - 1) / TB * ((N + TB - 1) / TB) * 256; }

hipError_t gemm_f32(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s) {
  LaunchInfo info;
  info.name = "gemm_f32";
  info.flops = 2.0 * g.M * (double)g.N * g.K;
  info.bytes = 4.0 * ((double)g.M * g.K + (double)g.K * g.N + (double)g.M * g.N);
  hipError_t e = hipErrorInvalidValue;
  if (g.colsum != nullptr) return e;  // column sums ride on the 16-bit kernels only
  trace_begin(s);
  if (a_kcontig && !b_kcontig && epi == EPI_STORE) e = launch<true, false, EPI_STORE>(g, s);
  else if (a_kcontig && !b_kcontig && epi == EPI_BIAS_GELU) e = launch<true, false, EPI_BIAS_GELU>(g, s);
  else if (a_kcontig && b_kcontig && epi == EPI_STORE) e = launch<true, true, EPI_STORE>(g, s);
  else if (a_kcontig && b_kcontig && epi == EPI_DGELU) e = launch<true, true, EPI_DGELU>(g, s);
  else if (a_kcontig && b_kcontig && epi == EPI_DGELU_H && g.C2 != nullptr) e = launch<true, true, EPI_DGELU_H>(g, s);
  else if (!a_kcontig && !b_kcontig && epi == EPI_F32) e = launch<false, false, EPI_F32>(g, s);
  trace_end(s, info);
  return e;
}

}  // namespace tps
