// Sequence-parallel edge steps on a rank's share of the tokens (memory-bound):
//
// LayerNorm forward.  One workgroup (4 waves) per row; a thread owns the
// 8-element chunks c = tid + 256 k of the row and keeps up to LN_MAXC of them
// in registers, so the row is read from HBM once (longer rows re-read their
// extra chunks, from L2).  Mean, then the mean squared deviation (two passes
// over the registers), in fp32; the row's mean and 1/sqrt(var + eps) are saved.
//
// LayerNorm backward.  A workgroup (8 waves) takes rows blockIdx.x, blockIdx.x + grid, ...
// For each row it forms xhat and g = dY * gamma per owned chunk (kept in
// registers), reduces sum(g) and sum(g * xhat) over the row, and writes
//   dX = rstd * (g - mean(g) - xhat * mean(g * xhat));
// meanwhile it accumulates dgamma (dY * xhat) and dbeta (dY) for its columns
// in registers.  Each workgroup writes one partial row of each; a fixed-order
// pass adds the partial rows (no atomics: bitwise reproducible).
//
// Bias + dropout + residual.  out = residual + keep * (Y + b) * 1/(1-p) with
// the keep decision taken from Philox4x32-10 (Salmon et al., "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11: 10 rounds of two 32x32->64-bit
// multiplies by the published constants, key bumped by the published Weyl
// increments) on the element's counter, so the backward regenerates the mask
// instead of storing it.  A thread handles 8 consecutive elements: two Philox
// blocks (the offset is a multiple of 8).
#include "elem.h"
#include "side.h"
#include "sp_edge.h"

namespace tps {
namespace {

constexpr int LN_T = 256;       // forward: threads per row
constexpr int LN_MAXC = 6;      // forward: register-held 8-element chunks per thread (rows up to 12288 read once)
constexpr int LNB_T = 512;      // backward: threads per workgroup
constexpr int LNB_MAXC = 3;     // backward: register-held chunks per thread (rows up to 12288)

// Sums over the workgroup (W waves), the same values in every thread; `red` is
// 2 W floats of LDS.  The wave sums are added in a fixed order.
template <int W>
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    a += __shfl_xor(a, m);
    b += __shfl_xor(b, m);
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();  // the previous use of red is finished
  if ((threadIdx.x & 63) == 0) {
    red[w] = a;
    red[W + w] = b;
  }
  __syncthreads();
  a = red[0];
  b = red[W];
#pragma unroll
  for (int i = 1; i < W; ++i) {
    a += red[i];
    b += red[W + i];
  }
}

template <typename T>
__global__ void __launch_bounds__(LN_T) layernorm_fwd_kernel(const void* X, const void* gamma, const void* beta,
                                                             void* Y, float* mean_out, float* rstd_out, int64_t h,
                                                             float eps) {
  __shared__ float red[8];
  const int64_t base = (int64_t)blockIdx.x * h;
  const int nch = (int)(h / 8);
  const float inv_h = 1.0f / (float)h;
  float v[LN_MAXC][8];
  float s = 0.0f, unused = 0.0f;
#pragma unroll
  for (int k = 0; k < LN_MAXC; ++k) {
    const int c = threadIdx.x + LN_T * k;
    if (c < nch) {
      load8<T>(X, base + 8 * c, v[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[k][e];
    }
  }
  for (int c = threadIdx.x + LN_T * LN_MAXC; c < nch; c += LN_T) {
    float t[8];
    load8<T>(X, base + 8 * c, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += t[e];
  }
  block_sum2<LN_T / 64>(s, unused, red);
  const float mean = s * inv_h;
  float q = 0.0f;
  unused = 0.0f;
#pragma unroll
  for (int k = 0; k < LN_MAXC; ++k) {
    const int c = threadIdx.x + LN_T * k;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[k][e] - mean;
        q += d * d;
      }
    }
  }
  for (int c = threadIdx.x + LN_T * LN_MAXC; c < nch; c += LN_T) {
    float t[8];
    load8<T>(X, base + 8 * c, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = t[e] - mean;
      q += d * d;
    }
  }
  block_sum2<LN_T / 64>(q, unused, red);
  const float rstd = 1.0f / sqrtf(q * inv_h + eps);
  auto emit = [&](int c, const float* x) {
    float g[8], bb[8] = {0, 0, 0, 0, 0, 0, 0, 0}, y[8];
    load8<T>(gamma, 8 * c, g);
    if (beta != nullptr) load8<T>(beta, 8 * c, bb);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (x[e] - mean) * rstd * g[e] + bb[e];
    store8<T>(Y, base + 8 * c, y);
  };
#pragma unroll
  for (int k = 0; k < LN_MAXC; ++k) {
    const int c = threadIdx.x + LN_T * k;
    if (c < nch) emit(c, v[k]);
  }
  for (int c = threadIdx.x + LN_T * LN_MAXC; c < nch; c += LN_T) {
    float x[8];
    load8<T>(X, base + 8 * c, x);
    emit(c, x);
  }
  if (threadIdx.x == 0 && mean_out != nullptr) {
    mean_out[blockIdx.x] = mean;
    rstd_out[blockIdx.x] = rstd;
  }
}

template <typename T>
__global__ void __launch_bounds__(LNB_T) layernorm_bwd_kernel(const void* X, const void* gamma, const float* mean,
                                                             const float* rstd, const void* dY, void* dX, float* part,
                                                             int64_t rows, int64_t h) {
  __shared__ float red[16];
  const int nch = (int)(h / 8);
  const float inv_h = 1.0f / (float)h;
  float* pg_row = part + (int64_t)blockIdx.x * h;                    // dgamma partial of this workgroup
  float* pb_row = part + ((int64_t)gridDim.x + blockIdx.x) * h;      // dbeta partial
  float pg[LNB_MAXC][8], pb[LNB_MAXC][8];
#pragma unroll
  for (int k = 0; k < LNB_MAXC; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) { pg[k][e] = 0.0f; pb[k][e] = 0.0f; }
  // columns past the register-held chunks accumulate in the partial rows
  for (int c = threadIdx.x + LNB_T * LNB_MAXC; c < nch; c += LNB_T)
#pragma unroll
    for (int e = 0; e < 8; ++e) { pg_row[8 * c + e] = 0.0f; pb_row[8 * c + e] = 0.0f; }

  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t base = row * h;
    const float mu = mean[row], r = rstd[row];
    float xh[LNB_MAXC][8], gy[LNB_MAXC][8];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < LNB_MAXC; ++k) {
      const int c = threadIdx.x + LNB_T * k;
      if (c < nch) {
        float x[8], dy[8], gm[8];
        load8<T>(X, base + 8 * c, x);
        load8<T>(dY, base + 8 * c, dy);
        load8<T>(gamma, 8 * c, gm);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xhat = (x[e] - mu) * r, g = dy[e] * gm[e];
          s1 += g;
          s2 += g * xhat;
          pg[k][e] += dy[e] * xhat;
          pb[k][e] += dy[e];
          xh[k][e] = xhat;
          gy[k][e] = g;
        }
      }
    }
    for (int c = threadIdx.x + LNB_T * LNB_MAXC; c < nch; c += LNB_T) {
      float x[8], dy[8], gm[8];
      load8<T>(X, base + 8 * c, x);
      load8<T>(dY, base + 8 * c, dy);
      load8<T>(gamma, 8 * c, gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xhat = (x[e] - mu) * r, g = dy[e] * gm[e];
        s1 += g;
        s2 += g * xhat;
        pg_row[8 * c + e] += dy[e] * xhat;
        pb_row[8 * c + e] += dy[e];
      }
    }
    block_sum2<LNB_T / 64>(s1, s2, red);
    const float a = s1 * inv_h, b = s2 * inv_h;
#pragma unroll
    for (int k = 0; k < LNB_MAXC; ++k) {
      const int c = threadIdx.x + LNB_T * k;
      if (c < nch) {
        float dx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) dx[e] = r * (gy[k][e] - a - xh[k][e] * b);
        store8<T>(dX, base + 8 * c, dx);
      }
    }
    for (int c = threadIdx.x + LNB_T * LNB_MAXC; c < nch; c += LNB_T) {
      float x[8], dy[8], gm[8], dx[8];
      load8<T>(X, base + 8 * c, x);
      load8<T>(dY, base + 8 * c, dy);
      load8<T>(gamma, 8 * c, gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) dx[e] = r * (dy[e] * gm[e] - a - (x[e] - mu) * r * b);
      store8<T>(dX, base + 8 * c, dx);
    }
  }
#pragma unroll
  for (int k = 0; k < LNB_MAXC; ++k) {
    const int c = threadIdx.x + LNB_T * k;
    if (c < nch) {
      *(f32x4*)(pg_row + 8 * c) = f32x4{pg[k][0], pg[k][1], pg[k][2], pg[k][3]};
      *(f32x4*)(pg_row + 8 * c + 4) = f32x4{pg[k][4], pg[k][5], pg[k][6], pg[k][7]};
      *(f32x4*)(pb_row + 8 * c) = f32x4{pb[k][0], pb[k][1], pb[k][2], pb[k][3]};
      *(f32x4*)(pb_row + 8 * c + 4) = f32x4{pb[k][4], pb[k][5], pb[k][6], pb[k][7]};
    }
  }
}

// Philox4x32-10 block for counter (c0, c1, 0, 0) under key (k0, k1).
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1, uint32_t* out) {
  uint32_t x0 = c0, x1 = c1, x2 = 0u, x3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // One 32 x 32 -> 64-bit multiply per product (v_mad_u64_u32) instead of
    // separate high and low halves.
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0, p1 = (uint64_t)0xCD9E8D57u * x2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
    x0 = n0;
    x1 = lo1;
    x2 = n2;
    x3 = lo0;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

// Keep decisions of the 8 elements starting at element e0 (a multiple of 8).
__device__ __forceinline__ void keep8(int64_t e0, uint64_t offset, uint64_t seed, uint64_t threshold, bool* keep) {
  const uint64_t blk = (offset + (uint64_t)e0) >> 2;   // even: offset and e0 are multiples of 8
  uint32_t w[8];
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), k0, k1, w);
  philox4x32_10((uint32_t)(blk + 1), (uint32_t)((blk + 1) >> 32), k0, k1, w + 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) keep[e] = (uint64_t)w[e] < threshold;
}

template <typename T>
__global__ void __launch_bounds__(256) bias_dropout_add_kernel(const void* Y, const void* b, const void* residual,
                                                               void* out, int64_t n8, int64_t h, uint64_t threshold,
                                                               float scale, uint64_t seed, uint64_t offset) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t e0 = 8 * i;
  float y[8], bb[8] = {0, 0, 0, 0, 0, 0, 0, 0}, r[8], o[8];
  bool keep[8];
  keep8(e0, offset, seed, threshold, keep);
  load8<T>(Y, e0, y);
  if (b != nullptr) load8<T>(b, e0 % h, bb);
  load8<T>(residual, e0, r);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = r[e] + (keep[e] ? (y[e] + bb[e]) * scale : 0.0f);
  store8<T>(out, e0, o);
}

template <typename T>
__global__ void __launch_bounds__(256) dropout_bwd_kernel(const void* dOut, void* dY, int64_t n8, uint64_t threshold,
                                                          float scale, uint64_t seed, uint64_t offset) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t e0 = 8 * i;
  float g[8], o[8];
  bool keep[8];
  keep8(e0, offset, seed, threshold, keep);
  load8<T>(dOut, e0, g);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = keep[e] ? g[e] * scale : 0.0f;
  store8<T>(dY, e0, o);
}

}  // namespace

int layernorm_fwd_threads() { return LN_T; }

int layernorm_bwd_chunks(int64_t rows) {
  int64_t c = (rows + 3) / 4;   // about 4 rows per workgroup, one workgroup per CU at most
  if (c > 256) c = 256;
  if (c < 1) c = 1;
  return (int)c;
}

hipError_t layernorm_fwd(const void* X, const void* gamma, const void* beta, void* Y, float* mean, float* rstd,
                         int64_t rows, int64_t h, float eps, Elem et, hipStream_t s) {
  const double el = elem_bytes(et);
  LaunchInfo info{"layernorm_fwd", 0.0, el * (2.0 * rows * h + (beta ? 2.0 : 1.0) * h) + (mean ? 8.0 * rows : 0.0)};
  const dim3 grid((unsigned)rows);
  trace_begin(s);
  if (et == ELEM_BF16)
    hipLaunchKernelGGL(layernorm_fwd_kernel<bf16>, grid, dim3(LN_T), 0, s, X, gamma, beta, Y, mean, rstd, h, eps);
  else if (et == ELEM_F16)
    hipLaunchKernelGGL(layernorm_fwd_kernel<f16>, grid, dim3(LN_T), 0, s, X, gamma, beta, Y, mean, rstd, h, eps);
  else
    hipLaunchKernelGGL(layernorm_fwd_kernel<float>, grid, dim3(LN_T), 0, s, X, gamma, beta, Y, mean, rstd, h, eps);
  trace_end(s, info);
  return hipGetLastError();
}

hipError_t layernorm_bwd(const void* X, const void* gamma, const float* mean, const float* rstd, const void* dY,
                         void* dX, float* dgamma, float* dbeta, float* ws, int accumulate, int64_t rows, int64_t h,
                         Elem et, hipStream_t s) {
  const int chunks = layernorm_bwd_chunks(rows);
  const double el = elem_bytes(et);
  LaunchInfo info{"layernorm_bwd", 0.0, el * (3.0 * rows * h + h) + 8.0 * rows + 8.0 * chunks * h};
  const dim3 grid((unsigned)chunks);
  trace_begin(s);
  if (et == ELEM_BF16)
    hipLaunchKernelGGL(layernorm_bwd_kernel<bf16>, grid, dim3(LNB_T), 0, s, X, gamma, mean, rstd, dY, dX, ws, rows, h);
  else if (et == ELEM_F16)
    hipLaunchKernelGGL(layernorm_bwd_kernel<f16>, grid, dim3(LNB_T), 0, s, X, gamma, mean, rstd, dY, dX, ws, rows, h);
  else
    hipLaunchKernelGGL(layernorm_bwd_kernel<float>, grid, dim3(LNB_T), 0, s, X, gamma, mean, rstd, dY, dX, ws, rows,
                       h);
  trace_end(s, info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dgamma and dbeta (when wanted) from their partial rows in one launch.
  return sum_partials(ws, dgamma, h, chunks, accumulate, "layernorm_bwd_finalize", s,
                      dbeta != nullptr ? ws + (int64_t)chunks * h : nullptr, dbeta);
}

hipError_t bias_dropout_add_fwd(const void* Y, const void* b, const void* residual, void* out, int64_t rows,
                                int64_t h, uint64_t threshold, float scale, uint64_t seed, uint64_t offset, Elem et,
                                hipStream_t s) {
  const int64_t n8 = rows * h / 8;
  LaunchInfo info{"bias_dropout_add", 0.0, elem_bytes(et) * (3.0 * rows * h + (b ? h : 0))};
  trace_begin(s);
  const dim3 grid((unsigned)((n8 + 255) / 256));
  if (et == ELEM_BF16)
    hipLaunchKernelGGL(bias_dropout_add_kernel<bf16>, grid, dim3(256), 0, s, Y, b, residual, out, n8, h, threshold,
                       scale, seed, offset);
  else if (et == ELEM_F16)
    hipLaunchKernelGGL(bias_dropout_add_kernel<f16>, grid, dim3(256), 0, s, Y, b, residual, out, n8, h, threshold,
                       scale, seed, offset);
  else
    hipLaunchKernelGGL(bias_dropout_add_kernel<float>, grid, dim3(256), 0, s, Y, b, residual, out, n8, h, threshold,
                       scale, seed, offset);
  trace_end(s, info);
  return hipGetLastError();
}

hipError_t dropout_bwd(const void* dOut, void* dY, int64_t rows, int64_t h, uint64_t threshold, float scale,
                       uint64_t seed, uint64_t offset, Elem et, hipStream_t s) {
  const int64_t n8 = rows * h / 8;
  LaunchInfo info{"dropout_bwd", 0.0, elem_bytes(et) * 2.0 * rows * h};
  trace_begin(s);
  const dim3 grid((unsigned)((n8 + 255) / 256));
  if (et == ELEM_BF16)
    hipLaunchKernelGGL(dropout_bwd_kernel<bf16>, grid, dim3(256), 0, s, dOut, dY, n8, threshold, scale, seed, offset);
  else if (et == ELEM_F16)
    hipLaunchKernelGGL(dropout_bwd_kernel<f16>, grid, dim3(256), 0, s, dOut, dY, n8, threshold, scale, seed, offset);
  else
    hipLaunchKernelGGL(dropout_bwd_kernel<float>, grid, dim3(256), 0, s, dOut, dY, n8, threshold, scale, seed, offset);
  trace_end(s, info);
  return hipGetLastError();
}

}  // namespace tps
