// Direct global -> LDS copies on gfx950 (buffer_load_dwordx4 ... lds) through a
// buffer resource whose record range zero-fills reads past the end of the data.
// Shared by the GEMM and the attention kernels.
#pragma once

#include "common.h"

namespace tps {

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// Direct global -> LDS copy of 16 bytes per lane: buffer_load_dwordx4 ... lds.
// Lane i's 16 bytes land at LDS byte address lds_addr + 16 i (lds_addr goes to
// M0 and must be wave-uniform); a lane whose offset is outside the buffer's
// record range writes zeros.  Issued as inline asm so that the compiler does not
// order every later LDS read behind the copy (it cannot tell which LDS bytes the
// copy writes); completion is awaited explicitly with vmcnt before the barrier
// that publishes the data.  M0 is not used for anything else in these kernels.
__device__ __forceinline__ void lds_dma16(const i32x4& rsrc, int voffset, unsigned lds_addr) {
  // One wait state between the M0 write and the LDS-DMA that reads it.
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voffset), "s"(rsrc)
               : "m0");
}

__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// A voffset at or beyond every record range: the lane reads zeros.
constexpr int OOB = 0x7ffffff0;

// Raw buffer resource over `bytes` bytes from `base` (wave-uniform arguments).
// The record count is capped at OOB, so an OOB offset always fails the range
// check, dword by dword; callers keep every in-range offset below the cap.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  const int64_t n = bytes < 0 ? 0 : (bytes > OOB ? OOB : bytes);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff));
  r[2] = __builtin_amdgcn_readfirstlane((int)n);
  r[3] = 0x00020000;
  return r;
}

// The same resource with a record count the caller has already clamped to
// [0, OOB] (wave-uniform), so that no 64-bit compare is made per copy.
__device__ __forceinline__ i32x4 make_rsrc_n(const void* base, int n) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff));
  r[2] = __builtin_amdgcn_readfirstlane(n);
  r[3] = 0x00020000;
  return r;
}

}  // namespace tps
