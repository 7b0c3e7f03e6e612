// Memory-bound side kernels: the token-sum of a gradient (bias gradients) and
// the unfused bias + GeLU pass.
//
// Column sum.  out[n] (+)= sum_t in[t, n] over a row-major [T x N] matrix.
// Pass 1: a workgroup (4 waves) owns 512 columns (a lane holds 8 consecutive
// columns, so each wave reads one contiguous 1 KiB (bf16) run of a row) and a
// chunk of rows; wave w sums rows w, w+4, ... of the chunk in fp32, the four
// wave sums are added in a fixed order through LDS and written as one partial
// row.  Pass 2 adds the partial rows of every column in a fixed order.  There
// are no atomics, so the result is bitwise reproducible.
//
// Bias + GeLU.  H = GeLU(Z + b) with 8 elements per lane (16-byte bf16 loads),
// the same GeLU evaluation as the GEMM epilogue (gelu.h).
#include "elem.h"
#include "gelu.h"
#include "side.h"

namespace tps {
namespace {

constexpr int CS_COLS = 512;  // columns per workgroup in pass 1
constexpr int CS_THREADS = 256;

template <typename E>
__global__ void __launch_bounds__(CS_THREADS) colsum_partial_kernel(const void* in, float* part, int64_t T,
                                                                    int64_t N, int64_t rows_per_chunk) {
  __shared__ float red[4][CS_COLS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * CS_COLS + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = min(T, r0 + rows_per_chunk);
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col < N) {
    // Rows r0 + wave, + 4, + 8, ... in that order; four loads in flight.
    int64_t r = r0 + wave;
    for (; r + 12 < r1; r += 16) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8<E>(in, (r + 4 * u) * N + col, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += v[u][e];
    }
    for (; r < r1; r += 4) {
      float v[8];
      load8<E>(in, r * N + col, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = s[e];
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = threadIdx.x + CS_THREADS * h;
    const int64_t gc = (int64_t)blockIdx.x * CS_COLS + c;
    if (gc < N) part[(int64_t)blockIdx.y * N + gc] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
  }
}

// Pass 2: a workgroup owns 64 columns (one per lane) of one of up to two
// (partial rows, output) pairs (blockIdx.y picks the pair).  Its 16 waves split
// the partial rows: wave w adds rows w, w + 16, w + 32, ... in that order, with
// up to 16 loads in flight before the adds (one round trip for 256 rows); the
// 16 wave sums are then added in a fixed order.
constexpr int FIN_WAVES = 16;

__global__ void __launch_bounds__(64 * FIN_WAVES) colsum_finalize_kernel(const float* part, float* out,
                                                                        const float* part2, float* out2, int64_t N,
                                                                        int chunks, int accumulate) {
  __shared__ float red[FIN_WAVES][64];
  if (blockIdx.y == 1) {
    part = part2;
    out = out2;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 64 + lane;
  float t = 0.0f;
  if (n < N) {
    int c = wave;
    for (; c + FIN_WAVES * 15 < chunks; c += FIN_WAVES * 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = part[(int64_t)(c + FIN_WAVES * u) * N + n];
#pragma unroll
      for (int u = 0; u < 16; ++u) t += v[u];
    }
    for (; c + FIN_WAVES * 3 < chunks; c += FIN_WAVES * 4) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = part[(int64_t)(c + FIN_WAVES * u) * N + n];
#pragma unroll
      for (int u = 0; u < 4; ++u) t += v[u];
    }
    for (; c < chunks; c += FIN_WAVES) t += part[(int64_t)c * N + n];
  }
  red[wave][lane] = t;
  __syncthreads();
  if (wave == 0 && n < N) {
    float sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < FIN_WAVES; ++w) sum += red[w][lane];
    out[n] = accumulate ? out[n] + sum : sum;
  }
}

template <typename E>
__global__ void __launch_bounds__(256) bias_gelu_kernel(const void* Z, const void* b, void* H, int64_t T,
                                                        int64_t N) {
  const int64_t nv = N / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * nv) return;
  const int64_t row = idx / nv;
  const int64_t c = (idx - row * nv) * 8;
  float z[8], bb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  load8<E>(Z, row * N + c, z);
  if (b != nullptr) load8<E>(b, c, bb);
  float h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = z[e] + bb[e];
    h[e] = gelu_f(x);
  }
  store8<E>(H, row * N + c, h);
}

// Loss-scaling check: g *= inv_scale over n fp32 values (4 per thread per
// step, grid-stride), and *found = 1 when any value is inf or NaN (one store
// per wave that saw one; the flag is never cleared here).
__global__ void __launch_bounds__(256) unscale_check_kernel(float* g, int64_t n, float inv_scale, int* found) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  bool bad = false;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      f32x4 v = *(f32x4*)(g + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bad |= !__builtin_isfinite(v[e]);
        v[e] *= inv_scale;
      }
      *(f32x4*)(g + i) = v;
    } else {
      for (int64_t k = i; k < n; ++k) {
        bad |= !__builtin_isfinite(g[k]);
        g[k] *= inv_scale;
      }
    }
  }
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) *found = 1;
}

}  // namespace

hipError_t unscale_check(float* g, int64_t n, float inv_scale, int* found, hipStream_t s) {
  int64_t blocks = (n + 1023) / 1024;
  if (blocks > 4096) blocks = 4096;
  LaunchInfo info{"unscale_check", 0.0, 8.0 * n};
  trace_begin(s);
  hipLaunchKernelGGL(unscale_check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g, n, inv_scale, found);
  trace_end(s, info);
  return hipGetLastError();
}

int colsum_chunks(int64_t T, int64_t N) {
  const int64_t col_blocks = (N + CS_COLS - 1) / CS_COLS;
  int64_t chunks = (1024 + col_blocks - 1) / col_blocks;
  const int64_t max_by_rows = (T + 3) / 4;
  if (chunks > max_by_rows) chunks = max_by_rows;
  if (chunks > 256) chunks = 256;
  if (chunks < 1) chunks = 1;
  return (int)chunks;
}

hipError_t colsum(const void* in, Elem el, float* out, float* ws, int accumulate, int64_t T, int64_t N,
                  hipStream_t s) {
  const int chunks = colsum_chunks(T, N);
  const int64_t rows_per_chunk = (T + chunks - 1) / chunks;
  const dim3 grid1((unsigned)((N + CS_COLS - 1) / CS_COLS), (unsigned)chunks);
  LaunchInfo info{"colsum_partial", 0.0, elem_bytes(el) * T * (double)N + 4.0 * chunks * (double)N};
  trace_begin(s);
  if (el == ELEM_BF16)
    hipLaunchKernelGGL(colsum_partial_kernel<bf16>, grid1, dim3(CS_THREADS), 0, s, in, ws, T, N, rows_per_chunk);
  else if (el == ELEM_F16)
    hipLaunchKernelGGL(colsum_partial_kernel<f16>, grid1, dim3(CS_THREADS), 0, s, in, ws, T, N, rows_per_chunk);
  else
    hipLaunchKernelGGL(colsum_partial_kernel<float>, grid1, dim3(CS_THREADS), 0, s, in, ws, T, N, rows_per_chunk);
  trace_end(s, info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  LaunchInfo info2{"colsum_finalize", 0.0, 4.0 * chunks * (double)N + 4.0 * (accumulate ? 2 : 1) * N};
  trace_begin(s);
  hipLaunchKernelGGL(colsum_finalize_kernel, dim3((unsigned)((N + 63) / 64)), dim3(64 * FIN_WAVES), 0, s,
                     (const float*)ws, out, (const float*)nullptr, (float*)nullptr, N, chunks, accumulate);
  trace_end(s, info2);
  return hipGetLastError();
}

hipError_t sum_partials(const float* part, float* out, int64_t N, int chunks, int accumulate, const char* name,
                        hipStream_t s, const float* part2, float* out2) {
  const int pairs = out2 != nullptr ? 2 : 1;
  LaunchInfo info{name, 0.0, pairs * (4.0 * chunks * (double)N + 4.0 * (accumulate ? 2 : 1) * N)};
  trace_begin(s);
  hipLaunchKernelGGL(colsum_finalize_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)pairs), dim3(64 * FIN_WAVES),
                     0, s, part, out, part2, out2, N, chunks, accumulate);
  trace_end(s, info);
  return hipGetLastError();
}

hipError_t bias_gelu(const void* Z, const void* b, void* H, Elem el, int64_t T, int64_t N, hipStream_t s) {
  const int64_t n = T * (N / 8);
  const dim3 grid((unsigned)((n + 255) / 256));
  LaunchInfo info{"bias_gelu", 0.0, elem_bytes(el) * (2.0 * T * (double)N + (b ? N : 0))};
  trace_begin(s);
  if (el == ELEM_BF16) hipLaunchKernelGGL(bias_gelu_kernel<bf16>, grid, dim3(256), 0, s, Z, b, H, T, N);
  else if (el == ELEM_F16) hipLaunchKernelGGL(bias_gelu_kernel<f16>, grid, dim3(256), 0, s, Z, b, H, T, N);
  else hipLaunchKernelGGL(bias_gelu_kernel<float>, grid, dim3(256), 0, s, Z, b, H, T, N);
  trace_end(s, info);
  return hipGetLastError();
}

}  // namespace tps
