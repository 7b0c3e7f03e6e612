// Memory-bound side kernels (elementwise.hip) and the matrix-core probe
// (probe.hip).
#pragma once

#include "common.h"

namespace tps {

// Column sum over rows (elementwise.hip): out[n] (+)= sum_t in[t, n].
// Uses `chunks * N` floats of workspace.
int colsum_chunks(int64_t T, int64_t N);
hipError_t colsum(const void* in, Elem el, float* out, float* ws, int accumulate,
                  int64_t T, int64_t N, hipStream_t s);

// out[n] (+)= sum over c < chunks of part[c * N + n], in a fixed order (elementwise.hip);
// with out2 given, the same for (part2, out2) in the same launch.
hipError_t sum_partials(const float* part, float* out, int64_t N, int chunks, int accumulate, const char* name,
                        hipStream_t s, const float* part2 = nullptr, float* out2 = nullptr);

// H = GeLU(Z + b) elementwise (elementwise.hip).
hipError_t bias_gelu(const void* Z, const void* b, void* H, Elem el, int64_t T, int64_t N, hipStream_t s);

// g[0..n) *= inv_scale; *found = 1 if any value is not finite (elementwise.hip).
hipError_t unscale_check(float* g, int64_t n, float inv_scale, int* found, hipStream_t s);

// Register-only MFMA throughput probe (probe.hip).
hipError_t mfma_probe(int blocks, int iters, float* sink, unsigned long long* ticks, hipStream_t s);

}  // namespace tps
