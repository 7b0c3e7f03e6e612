// 8-element vector loads and stores of bf16, fp16 or fp32 buffers through fp32
// registers (the memory-bound kernels' element access).
#pragma once

#include "common.h"

namespace tps {

template <typename T>
__device__ __forceinline__ void load8(const void* base, int64_t off, float* v) {
  if constexpr (sizeof(T) == 4) {
    const f32x4 a = *(const f32x4*)((const float*)base + off);
    const f32x4 b = *(const f32x4*)((const float*)base + off + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
    typedef __attribute__((__vector_size__(8 * sizeof(T)))) T v8;
    const v8 x = *(const v8*)((const T*)base + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
  }
}

template <typename T>
__device__ __forceinline__ void store8(void* base, int64_t off, const float* v) {
  if constexpr (sizeof(T) == 4) {
    float* p = (float*)base + off;
    *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    typedef __attribute__((__vector_size__(8 * sizeof(T)))) T v8;
    v8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (T)v[e];
    *(v8*)((T*)base + off) = x;
  }
}

inline double elem_bytes(Elem el) { return el == ELEM_F32 ? 4.0 : 2.0; }

}  // namespace tps
