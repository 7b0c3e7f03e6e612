// Core attention on one rank's local heads: for every head h and sequence b,
// O = softmax(Q K^T / sqrt(D) + M) V with M the causal mask (or none), bf16
// operands, fp32 scores and softmax, computed in one pass over the keys with a
// running maximum and sum (the exact IO-aware formulation: the T x T score
// matrix never reaches HBM).
//
// Forward kernel.  A workgroup owns 128 queries of one (sequence, head); each
// of its 4 waves owns 32 of them.  Keys and values stream through LDS in blocks
// of 64 (double-buffered, loaded through registers).  Per block a wave computes
// the transposed scores S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so that
// each lane holds 32 scores of ONE query (its column) and the softmax
// statistics (running max m, running sum l) are per-lane scalars; the two lanes
// that share a query (lane and lane ^ 32) combine their maxima with one swap.
// The probabilities then feed O^T += V^T P^T straight from registers: the
// MFMA's k index (keys) is a summation index, so the keys are fed in the order
// the score accumulators hold them (per lane half: 4 keys, skip 4, 4 keys) and
// the V^T operand is read from LDS with transposing reads in that same order.
// The O^T accumulator again has one query per lane, so the rescale by
// exp(m_old - m_new) is a per-lane multiply.
#include "attention.h"

#include <cmath>

namespace tps {
namespace {

constexpr int AW = 4;            // waves per workgroup
constexpr int QW = 32;           // queries per wave
constexpr int BQ = AW * QW;      // queries per workgroup
constexpr int BKEYS = 64;        // keys per LDS block
constexpr int NT = AW * 64;      // threads per workgroup

template <int D>
struct Shape {
  static constexpr int CH = D / 8;                      // 16-byte chunks per K/V row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int BLOCK_BYTES = BKEYS * ROW_BYTES;  // one K (or V) block
  static constexpr int LOADS = 2 * BKEYS * CH / NT;     // 16-byte loads per thread per K+V block
  static constexpr int KS = D / 16;                     // 16-wide d slices of a score product
  static constexpr int DT = D / 32;                     // 32-row d tiles of O^T
  static_assert(LOADS % 2 == 0 && (LOADS / 2) * NT == BKEYS * CH, "whole K and V loads per thread");
};

// LDS layouts of a block (rows = keys, 16-byte chunks XOR-permuted per row):
//  * K: chunk c of row r in slot c ^ (r mod CH).  A score operand read takes
//    one 16-byte chunk from 32 consecutive rows, which then fall in different
//    banks.
//  * V: chunk c of row r in slot c ^ (2 r mod CH).  A transposing read takes
//    8 bytes from each of 4 consecutive rows; the rows land 32 bytes apart.
template <int D>
__device__ __forceinline__ int k_slot(int c, int r) { return c ^ (r & (Shape<D>::CH - 1)); }
template <int D>
__device__ __forceinline__ int v_slot(int c, int r) { return c ^ ((2 * r) & (Shape<D>::CH - 1)); }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 4 consecutive bf16 of rows r0..r0+3, transposed: lane (16-lane group g, index
// i) supplies the address of row r0 + i/4, column c0 + 4 (i % 4); it receives
// column c0 + i of the 4 rows.
__device__ __forceinline__ bf16x4 read_tr(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
  return __builtin_bit_cast(bf16x4, v);
}

struct FwdArgs {
  const bf16* qkv;
  bf16* o;
  float* lse;
  int64_t T;
  int S, Hl, B, nqb, causal;
  float scale_log2;  // log2(e) / sqrt(D)
};

// Workgroup -> (query block, sequence, head).  The longest causal query blocks
// go first; workgroups of one (sequence, head) are B*Hl ids apart, so with B*Hl
// a multiple of 8 they share an XCD (and its L2 copy of K and V).
__device__ __forceinline__ void fwd_coords(const FwdArgs& a, int& qb, int& b, int& h) {
  const int bh = a.B * a.Hl;
  qb = a.nqb - 1 - (int)(blockIdx.x / bh);
  const int r = (int)(blockIdx.x % bh);
  b = r / a.Hl;
  h = r % a.Hl;
}

template <int D>
__global__ void __launch_bounds__(NT, 2) attn_fwd_kernel(FwdArgs a) {
  using SH = Shape<D>;
  __shared__ __attribute__((aligned(16))) char smem[2][2][SH::BLOCK_BYTES];  // [buffer][K, V]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  int qb, b, h;
  fwd_coords(a, qb, b, h);
  const int64_t ld = 3LL * a.Hl * D;
  const int64_t row0 = (int64_t)b * a.S;
  const bf16* qbase = a.qkv + row0 * ld + (int64_t)h * D;
  const bf16* kbase = qbase + (int64_t)a.Hl * D;
  const bf16* vbase = qbase + 2LL * a.Hl * D;
  const int q0 = qb * BQ;
  const int wq0 = q0 + wave * QW;          // first query of this wave
  const int qi = wq0 + l32;                // this lane's query
  const bool qvalid = qi < a.S;
  const int kend = a.causal ? min(a.S, q0 + BQ) : a.S;
  const int nkb = (kend + BKEYS - 1) / BKEYS;

  // Q operand (k = d, column = query), resident for the whole key loop.
  bf16x8 qf[SH::KS];
#pragma unroll
  for (int s = 0; s < SH::KS; ++s)
    qf[s] = qvalid ? *(const bf16x8*)(qbase + (int64_t)qi * ld + 16 * s + 8 * hh) : bf16x8{};

  bf16x8 stage[SH::LOADS];
  auto load_block = [&](int j) {
    const int k0 = j * BKEYS;
#pragma unroll
    for (int i = 0; i < SH::LOADS; ++i) {
      const int c = tid + NT * (i % (SH::LOADS / 2));
      const int r = c / SH::CH, ch = c % SH::CH;
      const bf16* src = (i < SH::LOADS / 2 ? kbase : vbase) + (int64_t)(k0 + r) * ld + ch * 8;
      stage[i] = (k0 + r < a.S) ? *(const bf16x8*)src : bf16x8{};
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < SH::LOADS; ++i) {
      const int c = tid + NT * (i % (SH::LOADS / 2));
      const int r = c / SH::CH, ch = c % SH::CH;
      if (i < SH::LOADS / 2)
        *(bf16x8*)(&smem[buf][0][r * SH::ROW_BYTES + k_slot<D>(ch, r) * 16]) = stage[i];
      else
        *(bf16x8*)(&smem[buf][1][r * SH::ROW_BYTES + v_slot<D>(ch, r) * 16]) = stage[i];
    }
  };

  // Transposing-read coordinates of this lane (16-lane group g = lane / 16:
  // lane half g / 2, column half g % 2).
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_r = 4 * (g16 >> 1) + (i16 >> 2);       // + 16 s (+ 8 for the second read)
  const int tr_c = 16 * (g16 & 1) + 4 * (i16 & 3);     // + 32 dt

  f32x16 oacc[SH::DT];
#pragma unroll
  for (int t = 0; t < SH::DT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  load_block(0);
  store_block(0);
  __syncthreads();
  for (int j = 0; j < nkb; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkb) load_block(j + 1);
    const char* Ks = smem[buf][0];
    const char* Vs = smem[buf][1];

    // S^T[key][query] for keys 32t + (0..31) of the block.
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < SH::KS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kr = 32 * t + l32;
        const bf16x8 kf = *(const bf16x8*)(Ks + kr * SH::ROW_BYTES + k_slot<D>(2 * s + hh, kr) * 16);
        sacc[t] = mfma(kf, qf[s], sacc[t]);
      }

    // Scale to log2 units, mask, block maximum of this lane's query.
    const int k0 = j * BKEYS;
    const bool masked = (k0 + BKEYS > a.S) || (a.causal && k0 + BKEYS - 1 > wq0);
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = sacc[t][v] * a.scale_log2;
        if (masked) {
          const int key = k0 + 32 * t + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key >= a.S || (a.causal && key > qi)) x = -INFINITY;
        }
        sacc[t][v] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);      // finite: key 0 is allowed for every query
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(sacc[t][v] - m_new);
        sacc[t][v] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < SH::DT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[t][v] *= alpha;

    // P^T as the B operand of 16-key slice s: k slot m of lane half hh is key
    // 16 s + 8 (m / 4) + 4 hh + m % 4, i.e. accumulator element 8 (s % 2) + m
    // of score tile s / 2.
    bf16x8 pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 8; ++m) pf[s][m] = (bf16)sacc[s >> 1][8 * (s & 1) + m];

    // O^T[d][query] += V^T P^T; V^T read with the same key order.
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < SH::DT; ++t) {
        const int col = 32 * t + tr_c;
        const int ra = 16 * s + tr_r, rb = ra + 8;
        const bf16x4 lo = read_tr(Vs + ra * SH::ROW_BYTES + v_slot<D>(col >> 3, ra) * 16 + (col & 7) * 2);
        const bf16x4 hi = read_tr(Vs + rb * SH::ROW_BYTES + v_slot<D>(col >> 3, rb) * 16 + (col & 7) * 2);
        bf16x8 vf;
        vf[0] = lo[0]; vf[1] = lo[1]; vf[2] = lo[2]; vf[3] = lo[3];
        vf[4] = hi[0]; vf[5] = hi[1]; vf[6] = hi[2]; vf[7] = hi[3];
        oacc[t] = mfma(vf, pf[s], oacc[t]);
      }

    if (j + 1 < nkb) store_block(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = 1.0f / l_tot;
    bf16* orow = a.o + (row0 + qi) * (int64_t)a.Hl * D + (int64_t)h * D;
#pragma unroll
    for (int t = 0; t < SH::DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (bf16)(oacc[t][4 * g + e] * inv);
        *(bf16x4*)(orow + 32 * t + 8 * g + 4 * hh) = o4;
      }
    if (a.lse != nullptr && hh == 0)
      a.lse[(int64_t)h * a.T + row0 + qi] = (m_run + __log2f(l_tot)) * 0.6931471805599453f;
  }
}

}  // namespace

double attention_fwd_flops(const AttnProblem& p) {
  const double S = p.S, B = (double)(p.T / p.S);
  const double pairs = p.causal ? S * (S + 1) / 2 : S * S;
  return 4.0 * p.D * pairs * B * p.Hl;
}

hipError_t attention_fwd(const bf16* qkv, bf16* o, float* lse, const AttnProblem& p, hipStream_t s) {
  FwdArgs a;
  a.qkv = qkv;
  a.o = o;
  a.lse = lse;
  a.T = p.T;
  a.S = p.S;
  a.Hl = p.Hl;
  a.B = (int)(p.T / p.S);
  a.nqb = (p.S + BQ - 1) / BQ;
  a.causal = p.causal ? 1 : 0;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p.D));
  const dim3 grid((unsigned)((int64_t)a.nqb * a.B * a.Hl));
  const double el = 2.0 * p.T * p.Hl * p.D;
  LaunchInfo info{p.D == 128 ? "attn_fwd_d128" : "attn_fwd_d64", attention_fwd_flops(p),
                  3.0 * el + el + (lse ? 4.0 * p.T * p.Hl : 0.0)};
  trace_begin(s);
  if (p.D == 128) hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, dim3(NT), 0, s, a);
  else hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(NT), 0, s, a);
  trace_end(s, info);
  return hipGetLastError();
}

hipError_t attention_bwd(const bf16*, const bf16*, const float*, const bf16*, bf16*, float*, const AttnProblem&,
                         hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace tps
