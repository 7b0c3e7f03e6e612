// bf16 GEMM with fused epilogues on the gfx950 matrix cores.
//
// C[M x N] = op(A)[M x K] * op(B)[K x N], fp32 accumulation in
// v_mfma_f32_32x32x16_bf16, one epilogue applied to the accumulators in
// registers before the only store (bias, bias + exact-erf GeLU with the
// pre-activation saved, GeLU' for the backward, or fp32 store / accumulate).
//
// Tiling.  A workgroup of 4 waves (2 x 2) owns a BM x BN tile of C; each wave a
// (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA blocks whose fp32 accumulators stay in
// the AGPR file for the whole K loop.  The K loop steps by 64 through two LDS
// stages: while the matrix cores work on one stage, the next A and B panels are
// copied HBM -> LDS by buffer_load_dwordx4 ... lds (no register staging; rows and
// columns outside the matrix read as zero through the buffer range check).  The
// MFMA operands of the next 16-wide k slice are read from LDS while the current
// slice's MFMAs issue (register double buffer).
//
// Layouts.  Each operand is kept in LDS in its memory orientation:
//  * K-contiguous panels (rows of A, or rows of B stored as [N x K]): a lane's
//    MFMA operand (8 consecutive k of one row) is one ds_read_b128;
//  * M/N-contiguous panels (A stored [K x M], B stored [K x N]): a lane's operand
//    is gathered across 8 k-rows by two ds_read_b64_tr_b16, whose 16-lane groups
//    transpose a 4 x 16 block.
//
// Output.  The MFMA is issued with the B fragment as its first operand, so a
// lane's 16 results of a block are 4 runs of 4 consecutive columns of one row
// of C: the epilogue loads bias / Z and stores 4 values at a time.
//
// Edges.  M, N and K may be ragged against the tile (T is arbitrary); loads
// outside the matrix read zero and stores outside it are skipped.  Feature
// dimensions are multiples of 8, so a 16-byte vector is entirely inside or
// entirely outside.
#include "common.h"

#include <string>

namespace tps {
namespace {

constexpr int KT = 32;        // K step per LDS stage
constexpr int GROUP_M = 8;    // tile rows per group in the tile order

__device__ __forceinline__ float gelu_f(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.7071067811865475f));
}

__device__ __forceinline__ float gelu_grad_f(float z) {
  const float cdf = 0.5f * (1.0f + erff(z * 0.7071067811865475f));
  const float pdf = 0.3989422804014327f * expf(-0.5f * z * z);
  return cdf + z * pdf;
}

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }

// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin,
// so consecutive ids are remapped to one XCD's contiguous range of logical
// tiles; logical tiles are ordered in groups of GROUP_M tile rows so that an
// XCD's workgroups share A and B panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = bid & 7;
  const int local = bid >> 3;
  const int base = total >> 3;
  const int rem = total & 7;
  const int logical = xcd * base + (xcd < rem ? xcd : rem) + local;
  const int per_group = GROUP_M * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Direct global -> LDS copy of 16 bytes per lane: buffer_load_dwordx4 ... lds.
// Lane i's 16 bytes land at LDS byte address lds_addr + 16 i (lds_addr goes to
// M0 and must be wave-uniform); a lane whose offset is outside the buffer's
// record range writes zeros.  Issued as inline asm so that the compiler does not
// order every later LDS read behind the copy (it cannot tell which LDS bytes the
// copy writes); completion is awaited explicitly with vmcnt before the barrier
// that publishes the stage.  M0 is not used for anything else in these kernels.
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

__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  // The record count is capped at 1 GiB: every in-range offset of one K step is
  // below that (feature dimensions are at most 2^21), and the OOB offset above it
  // then always fails the range check, dword by dword.
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x40000000 ? 0x40000000 : bytes);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff));
  r[2] = __builtin_amdgcn_readfirstlane((int)n);
  r[3] = 0x00020000;
  return r;
}

constexpr int OOB = 0x7ffffff0;  // a voffset beyond every record range: the lane reads zeros

template <int COLS>
__device__ __forceinline__ int mn_swz(int r) {
  return (COLS * 2) % 256 == 0 ? 4 * (r & 3) : 2 * (r & 3);
}

// LDS layouts (per stage, no padding; 16-byte chunks permuted by XOR so that the
// rows a read instruction touches fall in different banks):
//  * K-contiguous panel [rows][32]: 64-byte rows of 4 chunks; chunk c of row r
//    sits in slot c ^ ((r >> 2) & 3).
//  * M/N-contiguous panel [32][cols]: rows of 2*cols bytes; chunk c of k-row r sits
//    in slot c ^ mn_swz(r): 4 * (r & 3) when a row is a multiple of 256 bytes (the
//    four k-rows a transpose read touches would otherwise share banks), else
//    2 * (r & 3) (384-byte rows already alternate bank halves).  Either stays
//    inside the row.

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

template <int BM, int BN>
struct StageCfg {
  static constexpr int BYTES = (BM + BN) * KT * 2;
  static constexpr int N = (163840 / BYTES) < 5 ? (163840 / BYTES) : 5;  // LDS stages (<= 160 KiB)
};

// Wave roles.  A workgroup has 12 waves, 3 per SIMD: 8 consumer waves that read
// operands from LDS and issue the MFMAs (2 per SIMD, so one covers the other's
// LDS waits), and 4 producer waves that only issue the HBM -> LDS copies.  A
// copy instruction holds up its wave's instruction issue for tens of cycles;
// keeping them off the MFMA waves keeps the matrix pipe fed.
constexpr int N_CONS = 8;
constexpr int N_PROD = 4;
constexpr int NT_WS = 64 * (N_CONS + N_PROD);

// Consumer grid over the tile: CM x CN waves of (BM/CM) x (BN/CN) outputs.
template <int BM, int BN>
struct ConsCfg {
  static constexpr int CM = BM >= 256 ? 4 : 2;
  static constexpr int CN = N_CONS / CM;
  static constexpr int WM = BM / CM, WN = BN / CN;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "consumer tile must be whole 32x32 blocks");
};

template <int BM, int BN, bool AK, bool BKC, int EPI>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT_WS, NT_WS), amdgpu_waves_per_eu(3, 3)))
gemm_bf16_kernel(GemmArgs g) {
  constexpr int A_BYTES = BM * KT * 2;
  constexpr int B_BYTES = BN * KT * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int NSTAGE = StageCfg<BM, BN>::N;
  constexpr int A_INS = A_BYTES / 1024 / N_PROD;  // 1 KiB copies per producer wave per stage
  constexpr int B_INS = B_BYTES / 1024 / N_PROD;
  constexpr int NVM = A_INS + B_INS;
  constexpr int WM = ConsCfg<BM, BN>::WM, WN = ConsCfg<BM, BN>::WN, CN = ConsCfg<BM, BN>::CN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int KROW = KT * 2;               // bytes per row of a K-contiguous panel
  constexpr int KCH = KT / 8;                // 16-byte chunks per such row
  constexpr int PREF = NSTAGE - 1;           // K steps in flight ahead of the one computed
  static_assert(A_INS * N_PROD * 1024 == A_BYTES && B_INS * N_PROD * 1024 == B_BYTES, "whole copies");
  static_assert(NSTAGE >= 3, "need at least three stages");
  static_assert((PREF - 1) * NVM <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int nk = (g.K + KT - 1) / KT;

  if (wave >= N_CONS) {
    // ------------------------------------------------------------ producer
    const int pw = wave - N_CONS;
    const char* a_base = (const char*)g.A + 2 * (AK ? (int64_t)m0 * g.lda : (int64_t)m0);
    const char* b_base = (const char*)g.B + 2 * (BKC ? (int64_t)n0 * g.ldb : (int64_t)n0);
    const int64_t a_total = 2 * ((AK ? (int64_t)g.M : (int64_t)g.K) * g.lda - (AK ? (int64_t)m0 * g.lda : m0));
    const int64_t b_total = 2 * ((BKC ? (int64_t)g.N : (int64_t)g.K) * g.ldb - (BKC ? (int64_t)n0 * g.ldb : n0));
    const int64_t a_step = AK ? 2 * KT : 2 * (int64_t)KT * g.lda;
    const int64_t b_step = BKC ? 2 * KT : 2 * (int64_t)KT * g.ldb;

    // Per-lane byte offsets of each copy inside the tile at the current K step.
    int a_off[A_INS], a_kc[A_INS];
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
      const int q = (pw * A_INS + j) * 64 + lane;  // 16-byte chunk index in the stage's A panel
      if (AK) {
        const int r = q / KCH, sl = q % KCH, c = sl ^ ((r >> 2) & 3);
        a_off[j] = r * (int)g.lda * 2 + c * 16;
        a_kc[j] = c * 8;
      } else {
        constexpr int CPR = BM / 8;
        const int r = q / CPR, sl = q % CPR, c = sl ^ mn_swz<BM>(r);
        a_off[j] = (m0 + c * 8 < g.M) ? r * (int)g.lda * 2 + c * 16 : OOB;
        a_kc[j] = 0;
      }
    }
    int b_off[B_INS], b_kc[B_INS];
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      const int q = (pw * B_INS + j) * 64 + lane;
      if (BKC) {
        const int r = q / KCH, sl = q % KCH, c = sl ^ ((r >> 2) & 3);
        b_off[j] = r * (int)g.ldb * 2 + c * 16;
        b_kc[j] = c * 8;
      } else {
        constexpr int CPR = BN / 8;
        const int r = q / CPR, sl = q % CPR, c = sl ^ mn_swz<BN>(r);
        b_off[j] = (n0 + c * 8 < g.N) ? r * (int)g.ldb * 2 + c * 16 : OOB;
        b_kc[j] = 0;
      }
    }
    const unsigned smem_addr = lds_address(smem);
    // All copies of K step kt into LDS stage kt % NSTAGE (past the last step the
    // copies read only zeros into a stage that is not used again).
    auto issue_step = [&](int kt) {
      const int k0 = kt * KT;
      const unsigned st = smem_addr + (unsigned)((kt % NSTAGE) * STAGE);
      const i32x4 ra = make_rsrc(a_base + kt * a_step, a_total - kt * a_step);
      const i32x4 rb = make_rsrc(b_base + kt * b_step, b_total - kt * b_step);
#pragma unroll
      for (int j = 0; j < A_INS; ++j)
        lds_dma16(ra, (AK && k0 + a_kc[j] >= g.K) ? OOB : a_off[j], st + (pw * A_INS + j) * 1024);
#pragma unroll
      for (int j = 0; j < B_INS; ++j)
        lds_dma16(rb, (BKC && k0 + b_kc[j] >= g.K) ? OOB : b_off[j], st + A_BYTES + (pw * B_INS + j) * 1024);
    };
#pragma unroll
    for (int p = 0; p < PREF; ++p) issue_step(p);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((PREF - 1) * NVM));  // step 0 landed
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      issue_step(kt + PREF);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((PREF - 1) * NVM));  // step kt+1 landed
      __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no copy into this workgroup's LDS outlives it
    return;
  }

  // -------------------------------------------------------------- consumer
  const int wm = wave / CN;
  const int wn = wave % CN;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int kswz = (l32 >> 2) & 3;             // K-contig slot swizzle of this lane's row
  const int grp = lane >> 4, i16 = lane & 15;  // transpose read: 16-lane group, lane in it
  const int tr_row = 8 * (grp >> 1) + (i16 >> 2);
  const int tr_col = 16 * (grp & 1) + 4 * (i16 & 3);
  const int tr_swz_a = mn_swz<BM>(i16 >> 2);
  const int tr_swz_b = mn_swz<BN>(i16 >> 2);

  auto frag_k = [&](const char* panel, int row0, int s) -> bf16x8 {
    const int r = row0 + l32;
    const int slot = (2 * s + hi) ^ kswz;
    return *(const bf16x8*)(panel + r * KROW + slot * 16);
  };
  auto frag_mn = [&](const char* panel, int row_bytes, int swz, int col0, int s) -> bf16x8 {
    const int col = col0 + tr_col;
    const int slot = (col >> 3) ^ swz;
    const char* p0 = panel + (16 * s + tr_row) * row_bytes + slot * 16 + (col & 7) * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    const i16x4 hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p0 + 4 * row_bytes));
    const bf16x4 lo_b = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 hi_b = __builtin_bit_cast(bf16x4, hv);
    bf16x8 v;
    v[0] = lo_b[0]; v[1] = lo_b[1]; v[2] = lo_b[2]; v[3] = lo_b[3];
    v[4] = hi_b[0]; v[5] = hi_b[1]; v[6] = hi_b[2]; v[7] = hi_b[3];
    return v;
  };
  auto load_frags = [&](int kt, int s, bf16x8* fa, bf16x8* fb) {
    const char* sa = smem + (kt % NSTAGE) * STAGE;
    const char* sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = AK ? frag_k(sa, wm * WM + 32 * i, s) : frag_mn(sa, BM * 2, tr_swz_a, wm * WM + 32 * i, s);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = BKC ? frag_k(sb, wn * WN + 32 * j, s) : frag_mn(sb, BN * 2, tr_swz_b, wn * WN + 32 * j, s);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  constexpr int NS = KT / 16;           // 16-wide k slices per stage
  constexpr int LB = (NS - 1) & 1;      // operand buffer of the last slice
  constexpr int FM_HALF = FM / 2 > 0 ? FM / 2 : 1;
  auto mfma_rows = [&](const bf16x8* fa_, const bf16x8* fb_, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb_[j], fa_[i], acc[i][j], 0, 0, 0);
  };

  __syncthreads();  // step 0 is in LDS
  bf16x8 fa[2][FM], fb[2][FN];
  load_frags(0, 0, fa[0], fb[0]);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      load_frags(kt, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
      mfma_rows(fa[s & 1], fb[s & 1], 0, FM);
    }
    // Last slice: part of its MFMAs, the barrier that publishes step kt+1 (and
    // releases step kt's stage to the producers), then step kt+1's first
    // operands are read while the rest run.
    mfma_rows(fa[LB], fb[LB], 0, FM_HALF);
    __syncthreads();
    load_frags(kt + 1, 0, fa[LB ^ 1], fb[LB ^ 1]);
    mfma_rows(fa[LB], fb[LB], FM_HALF, FM);
  }

  // Epilogue.  Block (i, j), lane: row m = l32, columns 8q + 4*(lane/32) + 0..3.
  // The coordinates are passed through empty asm so that the compiler derives the
  // epilogue addresses here instead of hoisting them above the K loop, where they
  // would hold registers for its whole duration.
  int e_lane = lane, e_m0 = m0, e_n0 = n0, e_wave = wave;
  asm volatile("" : "+v"(e_lane));
  asm volatile("" : "+s"(e_m0), "+s"(e_n0), "+s"(e_wave));
  const int e_l32 = e_lane & 31;
  const int col_lane = 4 * (e_lane >> 5);
  const int e_wm = e_wave / CN, e_wn = e_wave % CN;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = e_m0 + e_wm * WM + 32 * i + e_l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = e_n0 + e_wn * WN + 32 * j + 8 * q + col_lane;
        if (n >= g.N) continue;
        float v[4] = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
        if (EPI == EPI_F32) {
          float* c = (float*)g.C + (int64_t)m * g.ldc + n;
          f32x4 o = {v[0], v[1], v[2], v[3]};
          if (g.accumulate) {
            const f32x4 old = *(const f32x4*)c;
            o[0] += old[0]; o[1] += old[1]; o[2] += old[2]; o[3] += old[3];
          }
          *(f32x4*)c = o;
        } else {
          if ((EPI == EPI_STORE || EPI == EPI_BIAS_GELU) && g.bias != nullptr) {
            const bf16x4 b = *(const bf16x4*)((const bf16*)g.bias + n);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += bf2f(b[e]);
          }
          if (EPI == EPI_BIAS_GELU && g.C2 != nullptr) {
            bf16x4 z;
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = (bf16)v[e];
            *(bf16x4*)((bf16*)g.C2 + (int64_t)m * g.ldc2 + n) = z;
          }
          if (EPI == EPI_BIAS_GELU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu_f(v[e]);
          }
          if (EPI == EPI_DGELU) {
            const bf16x4 z = *(const bf16x4*)((const bf16*)g.aux + (int64_t)m * g.ldaux + n);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= gelu_grad_f(bf2f(z[e]));
          }
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          *(bf16x4*)((bf16*)g.C + (int64_t)m * g.ldc + n) = o;
        }
      }
    }
  }
}

template <int BM, int BN, bool AK, bool BKC, int EPI>
const char* kname() {
  static const std::string s = std::string("gemm_bf16_") + (AK ? "n" : "t") + (BKC ? "t" : "n") + "_" +
                               (EPI == EPI_STORE ? "store" : EPI == EPI_BIAS_GELU ? "bias_gelu"
                                : EPI == EPI_DGELU ? "dgelu" : "f32") +
                               "_" + std::to_string(BM) + "x" + std::to_string(BN);
  return s.c_str();
}

template <int BM, int BN, bool AK, bool BKC, int EPI>
hipError_t launch_tile(const GemmArgs& g, hipStream_t s, const char** name) {
  *name = kname<BM, BN, AK, BKC, EPI>();
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AK, BKC, EPI>), dim3(tiles), dim3(NT_WS), 0, s, g);
  return hipGetLastError();
}

// Tile shape: the one with the least estimated time, counting whole waves of
// tiles over the 256 CUs (one workgroup per CU) and the lower MFMA efficiency
// of smaller tiles.
struct TileChoice { int bm, bn; };

TileChoice choose_tile(int M, int N) {
  static const struct { int bm, bn; double eff; } cand[] = {
      {256, 192, 1.00}, {192, 256, 1.00}, {256, 128, 0.92}, {128, 256, 0.92}, {128, 128, 0.75}};
  double best = 1e300;
  TileChoice pick = {256, 192};
  for (const auto& c : cand) {
    const long tiles = (long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const long waves = (tiles + 255) / 256;
    const double t = (double)waves * c.bm * c.bn / c.eff;
    if (t < best * 0.999) { best = t; pick = {c.bm, c.bn}; }
  }
  return pick;
}

template <bool AK, bool BKC, int EPI>
hipError_t launch_shape(const GemmArgs& g, hipStream_t s, const char** name) {
  const TileChoice t = choose_tile(g.M, g.N);
  if (t.bm == 256 && t.bn == 192) return launch_tile<256, 192, AK, BKC, EPI>(g, s, name);
  if (t.bm == 192 && t.bn == 256) return launch_tile<192, 256, AK, BKC, EPI>(g, s, name);
  if (t.bm == 256 && t.bn == 128) return launch_tile<256, 128, AK, BKC, EPI>(g, s, name);
  if (t.bm == 128 && t.bn == 256) return launch_tile<128, 256, AK, BKC, EPI>(g, s, name);
  return launch_tile<128, 128, AK, BKC, EPI>(g, s, name);
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s) {
  LaunchInfo info;
  info.name = "gemm_bf16";
  info.flops = 2.0 * g.M * (double)g.N * g.K;
  const double out_bytes = (epi == EPI_F32 ? 4.0 * (g.accumulate ? 2 : 1) : 2.0) * g.M * (double)g.N;
  info.bytes = 2.0 * ((double)g.M * g.K + (double)g.K * g.N) + out_bytes +
               ((epi == EPI_BIAS_GELU && g.C2) ? 2.0 * g.M * (double)g.N : 0.0) +
               (epi == EPI_DGELU ? 2.0 * g.M * (double)g.N : 0.0);
  // Instantiated layout / epilogue pairs: forward (NN), data gradient (NT) and
  // weight gradient (TN).
  hipError_t e = hipErrorInvalidValue;
  trace_begin(s);
  if (a_kcontig && !b_kcontig && epi == EPI_STORE) e = launch_shape<true, false, EPI_STORE>(g, s, &info.name);
  else if (a_kcontig && !b_kcontig && epi == EPI_BIAS_GELU) e = launch_shape<true, false, EPI_BIAS_GELU>(g, s, &info.name);
  else if (a_kcontig && b_kcontig && epi == EPI_STORE) e = launch_shape<true, true, EPI_STORE>(g, s, &info.name);
  else if (a_kcontig && b_kcontig && epi == EPI_DGELU) e = launch_shape<true, true, EPI_DGELU>(g, s, &info.name);
  else if (!a_kcontig && !b_kcontig && epi == EPI_F32) e = launch_shape<false, false, EPI_F32>(g, s, &info.name);
  trace_end(s, info);
  return e;
}

}  // namespace tps
