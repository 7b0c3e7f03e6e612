// Sequence-parallel edge steps on a rank's rows (sp_edge.hip): LayerNorm and
// bias + dropout + residual add, forward and backward.
#pragma once

#include "common.h"

namespace tps {

// Work-items of the LayerNorm forward's one workgroup per row.
int layernorm_fwd_threads();

// Workgroups (and partial rows of the parameter gradients) of the LayerNorm backward.
int layernorm_bwd_chunks(int64_t rows);

hipError_t layernorm_fwd(const void* X, const void* gamma, const void* beta, void* Y, float* mean, float* rstd,
                         int64_t rows, int64_t h, float eps, Elem el, hipStream_t s);
// ws: 2 * layernorm_bwd_chunks(rows) * h floats.
hipError_t layernorm_bwd(const void* X, const void* gamma, const float* mean, const float* rstd, const void* dY,
                         void* dX, float* dgamma, float* dbeta, float* ws, int accumulate, int64_t rows, int64_t h,
                         Elem el, hipStream_t s);

// Dropout keep rule: element e (row-major, plus offset) is kept when word
// (offset + e) mod 4 of Philox4x32-10(counter = (offset + e) / 4, key = seed)
// is below `threshold` (2^32 keeps everything).
hipError_t bias_dropout_add_fwd(const void* Y, const void* b, const void* residual, void* out, int64_t rows,
                                int64_t h, uint64_t threshold, float scale, uint64_t seed, uint64_t offset, Elem el,
                                hipStream_t s);
hipError_t dropout_bwd(const void* dOut, void* dY, int64_t rows, int64_t h, uint64_t threshold, float scale,
                       uint64_t seed, uint64_t offset, Elem el, hipStream_t s);

}  // namespace tps
