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
typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

// Element type of an activation / weight buffer (the C ABI's dtype codes).
enum Elem : int { ELEM_BF16 = 0, ELEM_F32 = 1, ELEM_F16 = 2 };

// Kernel launch record for the optional event trace.
struct LaunchInfo {
  const char* name;
  double flops;
  double bytes;
};

// Trace hooks (api.cpp). begin/end bracket a launch on `stream`.
void trace_begin(hipStream_t stream);
void trace_end(hipStream_t stream, const LaunchInfo& info);

}  // namespace tps
