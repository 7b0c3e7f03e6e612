// bf16 GEMM with fused epilogues on the gfx950 matrix cores.
//
// C[M x N] = op(A)[M x K] * op(B)[K x N], fp32 accumulation in
// v_mfma_f32_32x32x16_bf16, one epilogue applied to the accumulators in
// registers before the only store (bias, bias + exact-erf GeLU with the
// pre-activation saved, GeLU' for the backward, or fp32 store / accumulate).
//
// Tiling.  A workgroup of 4 waves (2 x 2) owns a BM x BN tile of C; each wave a
// (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA blocks whose fp32 accumulators stay in
// the AGPR file for the whole K loop.  The K loop steps by 64: the next A and B
// panels are fetched from HBM into registers with 16-byte loads while the matrix
// cores work on the current panels in LDS, then written to the other LDS buffer
// (two buffers, one barrier per step).
//
// Layouts.  Each operand is kept in LDS in its memory orientation:
//  * K-contiguous panels (rows of A, or rows of B stored as [N x K]) as
//    [rows][64 + 8] bf16; a lane's MFMA operand (8 consecutive k of one row) is
//    one ds_read_b128.
//  * M/N-contiguous panels (A stored [K x M], B stored [K x N]) as
//    [64][cols + 32] bf16; a lane's operand is gathered across 8 k-rows by two
//    ds_read_b64_tr_b16, whose 16-lane groups transpose a 4 x 16 block.
// The row pads put the rows a read touches in distinct LDS banks.
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

constexpr int KT = 64;        // K step per LDS stage
constexpr int NT = 256;       // threads per workgroup (4 waves)
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

template <int BM, int BN, bool AK, bool BKC, int EPI>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
gemm_bf16_kernel(GemmArgs g) {
  constexpr int A_LD = AK ? (KT + 8) : (BM + 32);
  constexpr int B_LD = BKC ? (KT + 8) : (BN + 32);
  constexpr int A_ELEMS = AK ? BM * A_LD : KT * A_LD;
  constexpr int B_ELEMS = BKC ? BN * B_LD : KT * B_LD;
  constexpr int STAGE = A_ELEMS + B_ELEMS;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_CH = BM * KT / 8 / NT;  // 16-byte chunks per thread
  constexpr int B_CH = BN * KT / 8 / NT;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const bf16* __restrict__ Ag = (const bf16*)g.A;
  const bf16* __restrict__ Bg = (const bf16*)g.B;

  // Per-thread global pointers for the first K step and their fixed bounds.
  const bf16* a_ptr[A_CH];
  bool a_ok[A_CH];
  int a_k[A_CH];      // k index of the chunk at K step 0 (row for !AK, col for AK)
  int a_lds[A_CH];
#pragma unroll
  for (int p = 0; p < A_CH; ++p) {
    const int c = tid + NT * p;
    if (AK) {
      const int row = c >> 3, kc = c & 7;
      const int gm = m0 + row;
      a_ok[p] = gm < g.M;
      a_k[p] = kc * 8;
      a_ptr[p] = Ag + (int64_t)(a_ok[p] ? gm : 0) * g.lda + kc * 8;
      a_lds[p] = row * A_LD + kc * 8;
    } else {
      constexpr int CPR = BM / 8;
      const int krow = c / CPR, mc = c % CPR;
      const int gm = m0 + mc * 8;
      a_ok[p] = gm < g.M;
      a_k[p] = krow;
      a_ptr[p] = Ag + (int64_t)krow * g.lda + (a_ok[p] ? gm : 0);
      a_lds[p] = krow * A_LD + mc * 8;
    }
  }
  const bf16* b_ptr[B_CH];
  bool b_ok[B_CH];
  int b_k[B_CH];
  int b_lds[B_CH];
#pragma unroll
  for (int p = 0; p < B_CH; ++p) {
    const int c = tid + NT * p;
    if (BKC) {
      const int row = c >> 3, kc = c & 7;
      const int gn = n0 + row;
      b_ok[p] = gn < g.N;
      b_k[p] = kc * 8;
      b_ptr[p] = Bg + (int64_t)(b_ok[p] ? gn : 0) * g.ldb + kc * 8;
      b_lds[p] = row * B_LD + kc * 8;
    } else {
      constexpr int CPR = BN / 8;
      const int krow = c / CPR, nc = c % CPR;
      const int gn = n0 + nc * 8;
      b_ok[p] = gn < g.N;
      b_k[p] = krow;
      b_ptr[p] = Bg + (int64_t)krow * g.ldb + (b_ok[p] ? gn : 0);
      b_lds[p] = krow * B_LD + nc * 8;
    }
  }

  bf16x8 ra[A_CH], rb[B_CH];
  const bf16x8 zero8 = {};

  auto load_global = [&](int kt) {
    const int k0 = kt * KT;
#pragma unroll
    for (int p = 0; p < A_CH; ++p) {
      const int k = k0 + a_k[p];
      const int64_t off = AK ? (int64_t)k0 : (int64_t)k0 * g.lda;
      ra[p] = (a_ok[p] && k < g.K) ? *(const bf16x8*)(a_ptr[p] + off) : zero8;
    }
#pragma unroll
    for (int p = 0; p < B_CH; ++p) {
      const int k = k0 + b_k[p];
      const int64_t off = BKC ? (int64_t)k0 : (int64_t)k0 * g.ldb;
      rb[p] = (b_ok[p] && k < g.K) ? *(const bf16x8*)(b_ptr[p] + off) : zero8;
    }
  };
  auto store_lds = [&](int stage) {
    bf16* As = smem + stage * STAGE;
    bf16* Bs = As + A_ELEMS;
#pragma unroll
    for (int p = 0; p < A_CH; ++p) *(bf16x8*)(As + a_lds[p]) = ra[p];
#pragma unroll
    for (int p = 0; p < B_CH; ++p) *(bf16x8*)(Bs + b_lds[p]) = rb[p];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Lane -> operand coordinates inside a 32-wide MFMA block.
  const int l32 = lane & 31;
  const int khalf = (lane >> 5) * 8;          // K-contig: k offset of this lane's 8 values
  const int grp = lane >> 4, i16 = lane & 15; // transpose read: 16-lane group and lane in it
  const int tr_k = 8 * (grp >> 1) + (i16 >> 2);
  const int tr_c = 16 * (grp & 1) + 4 * (i16 & 3);

  auto read_frag_a = [&](const bf16* As, int i, int s) -> bf16x8 {
    if (AK) {
      return *(const bf16x8*)(As + (wm * WM + 32 * i + l32) * A_LD + 16 * s + khalf);
    } else {
      const bf16* p0 = As + (16 * s + tr_k) * A_LD + wm * WM + 32 * i + tr_c;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p0 + 4 * A_LD));
      bf16x8 v;
      const bf16x4 lo_b = __builtin_bit_cast(bf16x4, lo);
      const bf16x4 hi_b = __builtin_bit_cast(bf16x4, hi);
      v[0] = lo_b[0]; v[1] = lo_b[1]; v[2] = lo_b[2]; v[3] = lo_b[3];
      v[4] = hi_b[0]; v[5] = hi_b[1]; v[6] = hi_b[2]; v[7] = hi_b[3];
      return v;
    }
  };
  auto read_frag_b = [&](const bf16* Bs, int j, int s) -> bf16x8 {
    if (BKC) {
      return *(const bf16x8*)(Bs + (wn * WN + 32 * j + l32) * B_LD + 16 * s + khalf);
    } else {
      const bf16* p0 = Bs + (16 * s + tr_k) * B_LD + wn * WN + 32 * j + tr_c;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p0 + 4 * B_LD));
      bf16x8 v;
      const bf16x4 lo_b = __builtin_bit_cast(bf16x4, lo);
      const bf16x4 hi_b = __builtin_bit_cast(bf16x4, hi);
      v[0] = lo_b[0]; v[1] = lo_b[1]; v[2] = lo_b[2]; v[3] = lo_b[3];
      v[4] = hi_b[0]; v[5] = hi_b[1]; v[6] = hi_b[2]; v[7] = hi_b[3];
      return v;
    }
  };

  const int nk = (g.K + KT - 1) / KT;
  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global(kt + 1);
    const bf16* As = smem + cur * STAGE;
    const bf16* Bs = As + A_ELEMS;
#pragma unroll
    for (int s = 0; s < KT / 16; ++s) {
      bf16x8 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = read_frag_a(As, i, s);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = read_frag_b(Bs, j, s);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Block (i, j), lane: row m = l32, columns 8q + 4*(lane/32) + 0..3.
  const int col_lane = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WM + 32 * i + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WN + 32 * j + 8 * q + col_lane;
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
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AK, BKC, EPI>), dim3(tiles), dim3(NT), 0, s, g);
  return hipGetLastError();
}

// Tile shape: the one with the least estimated time, counting whole waves of
// tiles over the 256 CUs (one workgroup per CU) and the lower MFMA efficiency
// of smaller tiles.
struct TileChoice { int bm, bn; };

TileChoice choose_tile(int M, int N) {
  static const struct { int bm, bn; double eff; } cand[] = {
      {256, 256, 1.00}, {256, 128, 0.88}, {128, 256, 0.88}, {128, 128, 0.72}};
  double best = 1e300;
  TileChoice pick = {256, 256};
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
  if (t.bm == 256 && t.bn == 256) return launch_tile<256, 256, AK, BKC, EPI>(g, s, name);
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
