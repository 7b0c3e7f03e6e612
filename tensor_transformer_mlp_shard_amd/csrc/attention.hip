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

// LDS layout of a block (rows = keys or queries, D bf16 each): 16-byte chunk c
// of row r sits in slot c ^ f(r), one permutation that keeps both kinds of
// operand read free of bank conflicts (64 banks of 4 bytes = 256 bytes):
//  * row reads (16 bytes per lane, chunk c of 16 consecutive rows): f takes 16
//    distinct values on 16 consecutive rows (D = 128; for D = 64, where two
//    rows share a 256-byte bank sweep, 8 distinct values on each row parity);
//  * transposing reads (8 bytes per lane; 32 lanes cover chunks 4j..4j+3 of rows
//    4i..4i+3): the four rows' 64-byte chunk groups land in four different
//    quarters of the bank sweep.
//  D = 128: f(r) = 4 (r mod 4) + (r / 4 mod 4);  D = 64: f(r) = 4 (r / 2 mod 2) + (r / 4 mod 4).
template <int D>
__device__ __forceinline__ int kv_slot(int c, int r) {
  return D == 128 ? c ^ (4 * (r & 3) + ((r >> 2) & 3)) : c ^ (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
}

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
        *(bf16x8*)(&smem[buf][0][r * SH::ROW_BYTES + kv_slot<D>(ch, r) * 16]) = stage[i];
      else
        *(bf16x8*)(&smem[buf][1][r * SH::ROW_BYTES + kv_slot<D>(ch, r) * 16]) = stage[i];
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

    // S^T[key][query] for keys 32t + (0..31) of the block; the operands of
    // slice s + 1 are read while the MFMAs of slice s run.
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    auto kfrag = [&](int s, int t) {
      const int kr = 32 * t + l32;
      return *(const bf16x8*)(Ks + kr * SH::ROW_BYTES + kv_slot<D>(2 * s + hh, kr) * 16);
    };
    bf16x8 kf[2][2];
    kf[0][0] = kfrag(0, 0);
    kf[0][1] = kfrag(0, 1);
#pragma unroll
    for (int s = 0; s < SH::KS; ++s) {
      if (s + 1 < SH::KS) {
        kf[(s + 1) & 1][0] = kfrag(s + 1, 0);
        kf[(s + 1) & 1][1] = kfrag(s + 1, 1);
      }
      sacc[0] = mfma(kf[s & 1][0], qf[s], sacc[0]);
      sacc[1] = mfma(kf[s & 1][1], qf[s], sacc[1]);
    }

    // Mask, block maximum of this lane's query (on the raw scores: the scale is
    // positive), then p = 2^(s * log2(e)/sqrt(D) - m) as one FMA and an exp2.
    const int k0 = j * BKEYS;
    const bool masked = (k0 + BKEYS > a.S) || (a.causal && k0 + BKEYS - 1 > wq0);
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if (masked) {
          const int key = k0 + 32 * t + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key >= a.S || (a.causal && key > qi)) sacc[t][v] = -INFINITY;
        }
        mloc = fmaxf(mloc, sacc[t][v]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc * a.scale_log2);   // finite: key 0 is allowed for every query
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][v], a.scale_log2, -m_new));
        sacc[t][v] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // The running maximum rarely moves after the first blocks: rescale O only
    // when it moved for some lane of the wave.
    if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
      for (int t = 0; t < SH::DT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[t][v] *= alpha;
    }

    // P^T as the B operand of 16-key slice s: k slot m of lane half hh is key
    // 16 s + 8 (m / 4) + 4 hh + m % 4, i.e. accumulator element 8 (s % 2) + m
    // of score tile s / 2.
    bf16x8 pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 8; ++m) pf[s][m] = (bf16)sacc[s >> 1][8 * (s & 1) + m];

    // O^T[d][query] += V^T P^T; V^T read with the same key order, one operand
    // ahead of the MFMA that uses it.
    auto vfrag = [&](int s, int t) {
      const int col = 32 * t + tr_c;
      const int ra = 16 * s + tr_r, rb = ra + 8;
      const bf16x4 lo = read_tr(Vs + ra * SH::ROW_BYTES + kv_slot<D>(col >> 3, ra) * 16 + (col & 7) * 2);
      const bf16x4 hi = read_tr(Vs + rb * SH::ROW_BYTES + kv_slot<D>(col >> 3, rb) * 16 + (col & 7) * 2);
      bf16x8 v;
      v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
      v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
      return v;
    };
    bf16x8 vf[2];
    vf[0] = vfrag(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < SH::DT; ++t) {
        const int n = s * SH::DT + t;
        if (n + 1 < 4 * SH::DT) vf[(n + 1) & 1] = vfrag((n + 1) / SH::DT, (n + 1) % SH::DT);
        oacc[t] = mfma(vf[n & 1], pf[s], oacc[t]);
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

// ---------------------------------------------------------------- backward
//
// With P the forward's probabilities (recomputed from the saved log-sum-exp),
// dP = dO V^T and Dt = rowsum(dO * O) = rowsum(P * dP):
//   dV = P^T dO,  dS = P * (dP - Dt),  dK = dS^T Q / sqrt(D),  dQ = dS K / sqrt(D).
// Three kernels, no atomics (bitwise reproducible):
//  * attn_bwd_dot: Dt for every (token, head);
//  * attn_bwd_dkdv: a workgroup owns 128 keys (32 per wave, one per lane
//    column); K and V of its keys stay in registers; queries stream through
//    LDS in blocks of 64.  Scores are computed as S[query][key] so each lane
//    holds one key's column, and P and dS feed dV^T += dO^T P and
//    dK^T += Q^T dS from registers (queries in the accumulator order, dO^T and
//    Q^T read from LDS with transposing reads in that order);
//  * attn_bwd_dq: a workgroup owns 128 queries (32 per wave, one per lane
//    column) as in the forward; keys and values stream through LDS in blocks
//    of 64; S^T and dP^T = V dO^T give dS^T, which feeds dQ^T += K^T dS^T.

struct BwdArgs {
  const bf16* qkv;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  float* dt;        // [Hl x T]
  bf16* dqkv;
  int64_t T;
  int S, Hl, B, nb, causal;  // nb: 128-row blocks per sequence
  float scale_log2;           // log2(e) / sqrt(D)
  float scale;                // 1 / sqrt(D)
};

constexpr float LOG2E = 1.4426950408889634f;

// Dt[h, t] = sum_d dO[t, h, d] * O[t, h, d]; D/8 lanes per (token, head) row.
template <int D>
__global__ void __launch_bounds__(NT) attn_bwd_dot_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t row = ((int64_t)blockIdx.x * NT + threadIdx.x) / LPR;   // token * Hl + head
  const int part = threadIdx.x % LPR;
  float s = 0.0f;
  if (row < a.T * a.Hl) {
    const bf16x8 o = *(const bf16x8*)(a.o + row * D + part * 8);
    const bf16x8 g = *(const bf16x8*)(a.dout + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)o[e] * (float)g[e];
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m);
  if (row < a.T * a.Hl && part == 0) {
    const int64_t t = row / a.Hl;
    const int h = (int)(row % a.Hl);
    a.dt[(int64_t)h * a.T + t] = s;
  }
}

// 16-byte operand of an MFMA from an LDS block: row r, 16-wide
// slice s, lane half hh (elements 16 s + 8 hh .. + 7).
template <int D>
__device__ __forceinline__ bf16x8 lds_row_frag(const char* blk, int r, int s, int hh) {
  return *(const bf16x8*)(blk + r * Shape<D>::ROW_BYTES + kv_slot<D>(2 * s + hh, r) * 16);
}

// Transposed operand from an LDS block: columns 32 t + (0..31)
// of rows 16 s + {4 hh + 0..3, 8 + 4 hh + 0..3} (the accumulator order).
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_frag(const char* blk, int t, int s, int tr_r, int tr_c) {
  const int col = 32 * t + tr_c;
  const int ra = 16 * s + tr_r, rb = ra + 8;
  const bf16x4 lo = read_tr(blk + ra * Shape<D>::ROW_BYTES + kv_slot<D>(col >> 3, ra) * 16 + (col & 7) * 2);
  const bf16x4 hi = read_tr(blk + rb * Shape<D>::ROW_BYTES + kv_slot<D>(col >> 3, rb) * 16 + (col & 7) * 2);
  bf16x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// Two 64-row blocks (rows r0.. of the sequence; base / row stride of each) into
// registers, zero past the sequence end, then into LDS (kv_slot layout).
template <int D>
struct PairStager {
  static constexpr int L = Shape<D>::LOADS;  // 16-byte loads per thread (both blocks)
  bf16x8 st[L];
  __device__ __forceinline__ void load(const bf16* base0, int64_t ld0, const bf16* base1, int64_t ld1, int r0, int S,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int c = tid + NT * (i % (L / 2));
      const int r = c / Shape<D>::CH, ch = c % Shape<D>::CH;
      const bf16* src = i < L / 2 ? base0 + (int64_t)(r0 + r) * ld0 + ch * 8 : base1 + (int64_t)(r0 + r) * ld1 + ch * 8;
      st[i] = (r0 + r < S) ? *(const bf16x8*)src : bf16x8{};
    }
  }
  __device__ __forceinline__ void store(char* blk0, char* blk1, int tid) const {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int c = tid + NT * (i % (L / 2));
      const int r = c / Shape<D>::CH, ch = c % Shape<D>::CH;
      *(bf16x8*)((i < L / 2 ? blk0 : blk1) + r * Shape<D>::ROW_BYTES + kv_slot<D>(ch, r) * 16) = st[i];
    }
  }
};

template <int D>
__global__ void __launch_bounds__(NT, 1) attn_bwd_dkdv_kernel(BwdArgs a) {
  using SH = Shape<D>;
  constexpr int QB = 64;  // queries per LDS block
  __shared__ __attribute__((aligned(16))) char smem[2][2][SH::BLOCK_BYTES];  // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float stat[2][2][QB];              // [buffer][lse2, Dt]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int bh = a.B * a.Hl;
  const int kb = (int)(blockIdx.x / bh);           // causal: low key blocks have the most queries
  const int b = (int)(blockIdx.x % bh) / a.Hl, h = (int)(blockIdx.x % bh) % a.Hl;
  const int64_t ld = 3LL * a.Hl * D;
  const int64_t row0 = (int64_t)b * a.S;
  const bf16* qbase = a.qkv + row0 * ld + (int64_t)h * D;
  const bf16* kbase = qbase + (int64_t)a.Hl * D;
  const bf16* vbase = qbase + 2LL * a.Hl * D;
  const bf16* dobase = a.dout + row0 * (int64_t)a.Hl * D + (int64_t)h * D;
  const int64_t ldo = (int64_t)a.Hl * D;
  const int kj = kb * 128 + wave * 32 + l32;      // this lane's key
  const bool kvalid = kj < a.S;

  // K and V of this lane's key as the B operand (k = d) of S and dP.
  bf16x8 kf[SH::KS], vf[SH::KS];
#pragma unroll
  for (int s = 0; s < SH::KS; ++s) {
    kf[s] = kvalid ? *(const bf16x8*)(kbase + (int64_t)kj * ld + 16 * s + 8 * hh) : bf16x8{};
    vf[s] = kvalid ? *(const bf16x8*)(vbase + (int64_t)kj * ld + 16 * s + 8 * hh) : bf16x8{};
  }
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_r = 4 * (g16 >> 1) + (i16 >> 2);
  const int tr_c = 16 * (g16 & 1) + 4 * (i16 & 3);

  f32x16 dk[SH::DT], dv[SH::DT];
#pragma unroll
  for (int t = 0; t < SH::DT; ++t) { dk[t] = f32x16{}; dv[t] = f32x16{}; }

  const int qstart = a.causal ? kb * 128 : 0;      // earlier queries see none of these keys
  const int nqblk = (a.S - qstart + QB - 1) / QB;
  PairStager<D> stg;
  auto load_stats = [&](int buf, int q0) {
    if (tid < QB) {
      const int q = q0 + tid;
      stat[buf][0][tid] = q < a.S ? a.lse[(int64_t)h * a.T + row0 + q] * LOG2E : INFINITY;
      stat[buf][1][tid] = q < a.S ? a.dt[(int64_t)h * a.T + row0 + q] : 0.0f;
    }
  };
  stg.load(qbase, ld, dobase, ldo, qstart, a.S, tid);
  stg.store(smem[0][0], smem[0][1], tid);
  load_stats(0, qstart);
  __syncthreads();
  for (int j = 0; j < nqblk; ++j) {
    const int buf = j & 1;
    const int q0 = qstart + j * QB;
    if (j + 1 < nqblk) stg.load(qbase, ld, dobase, ldo, q0 + QB, a.S, tid);
    const char* Qs = smem[buf][0];
    const char* Gs = smem[buf][1];

    // S[query][key] and dP[query][key] for queries 32 t + (0..31) of the block.
    f32x16 sc[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < SH::KS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[t] = mfma(lds_row_frag<D>(Qs, 32 * t + l32, s, hh), kf[s], sc[t]);
        dp[t] = mfma(lds_row_frag<D>(Gs, 32 * t + l32, s, hh), vf[s], dp[t]);
      }
    // P and dS; this lane's entries are queries 32 t + 8 g + 4 hh + e.
    const bool masked = a.causal && q0 < kb * 128 + wave * 32 + 31;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qo = 32 * t + 8 * g + 4 * hh;
        const f32x4 l2 = *(const f32x4*)&stat[buf][0][qo];
        const f32x4 dd = *(const f32x4*)&stat[buf][1][qo];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * g + e;
          float p = __builtin_amdgcn_exp2f(sc[t][v] * a.scale_log2 - l2[e]);
          if (masked && kj > q0 + qo + e) p = 0.0f;
          sc[t][v] = p;
          dp[t][v] = p * (dp[t][v] - dd[e]);
        }
      }
    bf16x8 pf[4], sf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        pf[s][m] = (bf16)sc[s >> 1][8 * (s & 1) + m];
        sf[s][m] = (bf16)dp[s >> 1][8 * (s & 1) + m];
      }
    // dV^T += dO^T P, dK^T += Q^T dS (k = the block's queries in accumulator order).
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < SH::DT; ++t) {
        dv[t] = mfma(lds_tr_frag<D>(Gs, t, s, tr_r, tr_c), pf[s], dv[t]);
        dk[t] = mfma(lds_tr_frag<D>(Qs, t, s, tr_r, tr_c), sf[s], dk[t]);
      }
    if (j + 1 < nqblk) {
      stg.store(smem[buf ^ 1][0], smem[buf ^ 1][1], tid);
      load_stats(buf ^ 1, q0 + QB);
    }
    __syncthreads();
  }

  if (kvalid) {
    bf16* krow = a.dqkv + (row0 + kj) * ld + (int64_t)a.Hl * D + (int64_t)h * D;
    bf16* vrow = krow + (int64_t)a.Hl * D;
#pragma unroll
    for (int t = 0; t < SH::DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = (bf16)(dk[t][4 * g + e] * a.scale);
          v4[e] = (bf16)dv[t][4 * g + e];
        }
        *(bf16x4*)(krow + 32 * t + 8 * g + 4 * hh) = k4;
        *(bf16x4*)(vrow + 32 * t + 8 * g + 4 * hh) = v4;
      }
  }
}

template <int D>
__global__ void __launch_bounds__(NT, 1) attn_bwd_dq_kernel(BwdArgs a) {
  using SH = Shape<D>;
  __shared__ __attribute__((aligned(16))) char smem[2][2][SH::BLOCK_BYTES];  // [buffer][K, V]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int bh = a.B * a.Hl;
  const int qb = a.nb - 1 - (int)(blockIdx.x / bh);  // longest causal query blocks first
  const int b = (int)(blockIdx.x % bh) / a.Hl, h = (int)(blockIdx.x % bh) % a.Hl;
  const int64_t ld = 3LL * a.Hl * D;
  const int64_t row0 = (int64_t)b * a.S;
  const bf16* qbase = a.qkv + row0 * ld + (int64_t)h * D;
  const bf16* kbase = qbase + (int64_t)a.Hl * D;
  const bf16* vbase = qbase + 2LL * a.Hl * D;
  const int64_t ldo = (int64_t)a.Hl * D;
  const bf16* dobase = a.dout + row0 * ldo + (int64_t)h * D;
  const int q0 = qb * BQ;
  const int wq0 = q0 + wave * QW;
  const int qi = wq0 + l32;
  const bool qvalid = qi < a.S;
  const int kend = a.causal ? min(a.S, q0 + BQ) : a.S;
  const int nkb = (kend + BKEYS - 1) / BKEYS;

  // Q and dO of this lane's query as the B operand (k = d) of S^T and dP^T.
  bf16x8 qf[SH::KS], gf[SH::KS];
#pragma unroll
  for (int s = 0; s < SH::KS; ++s) {
    qf[s] = qvalid ? *(const bf16x8*)(qbase + (int64_t)qi * ld + 16 * s + 8 * hh) : bf16x8{};
    gf[s] = qvalid ? *(const bf16x8*)(dobase + (int64_t)qi * ldo + 16 * s + 8 * hh) : bf16x8{};
  }
  const float lse2 = qvalid ? a.lse[(int64_t)h * a.T + row0 + qi] * LOG2E : INFINITY;
  const float dti = qvalid ? a.dt[(int64_t)h * a.T + row0 + qi] : 0.0f;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_r = 4 * (g16 >> 1) + (i16 >> 2);
  const int tr_c = 16 * (g16 & 1) + 4 * (i16 & 3);

  f32x16 dq[SH::DT];
#pragma unroll
  for (int t = 0; t < SH::DT; ++t) dq[t] = f32x16{};

  PairStager<D> stg;
  stg.load(kbase, ld, vbase, ld, 0, a.S, tid);
  stg.store(smem[0][0], smem[0][1], tid);
  __syncthreads();
  for (int j = 0; j < nkb; ++j) {
    const int buf = j & 1;
    const int k0 = j * BKEYS;
    if (j + 1 < nkb) stg.load(kbase, ld, vbase, ld, k0 + BKEYS, a.S, tid);
    const char* Ks = smem[buf][0];
    const char* Vs = smem[buf][1];

    // S^T[key][query] and dP^T[key][query] = (V dO^T) for keys 32 t + (0..31).
    f32x16 sc[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < SH::KS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[t] = mfma(lds_row_frag<D>(Ks, 32 * t + l32, s, hh), qf[s], sc[t]);
        dp[t] = mfma(lds_row_frag<D>(Vs, 32 * t + l32, s, hh), gf[s], dp[t]);
      }
    const bool masked = (k0 + BKEYS > a.S) || (a.causal && k0 + BKEYS - 1 > wq0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = __builtin_amdgcn_exp2f(sc[t][v] * a.scale_log2 - lse2);
        if (masked) {
          const int key = k0 + 32 * t + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key >= a.S || (a.causal && key > qi)) p = 0.0f;
        }
        dp[t][v] = p * (dp[t][v] - dti);
      }
    bf16x8 sf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 8; ++m) sf[s][m] = (bf16)dp[s >> 1][8 * (s & 1) + m];
    // dQ^T += K^T dS^T (k = the block's keys in accumulator order).
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < SH::DT; ++t) dq[t] = mfma(lds_tr_frag<D>(Ks, t, s, tr_r, tr_c), sf[s], dq[t]);
    if (j + 1 < nkb) stg.store(smem[buf ^ 1][0], smem[buf ^ 1][1], tid);
    __syncthreads();
  }

  if (qvalid) {
    bf16* qrow = a.dqkv + (row0 + qi) * ld + (int64_t)h * D;
#pragma unroll
    for (int t = 0; t < SH::DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 q4;
#pragma unroll
        for (int e = 0; e < 4; ++e) q4[e] = (bf16)(dq[t][4 * g + e] * a.scale);
        *(bf16x4*)(qrow + 32 * t + 8 * g + 4 * hh) = q4;
      }
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


hipError_t attention_bwd(const bf16* qkv, const bf16* o, const float* lse, const bf16* dout, bf16* dqkv,
                         float* ws, const AttnProblem& p, hipStream_t s) {
  BwdArgs a;
  a.qkv = qkv;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dt = ws;
  a.dqkv = dqkv;
  a.T = p.T;
  a.S = p.S;
  a.Hl = p.Hl;
  a.B = (int)(p.T / p.S);
  a.nb = (p.S + 127) / 128;
  a.causal = p.causal ? 1 : 0;
  a.scale = (float)(1.0 / std::sqrt((double)p.D));
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p.D));
  const double el = 2.0 * p.T * p.Hl * p.D;   // bytes of one [T x Hl*D] bf16 tensor
  const bool d128 = p.D == 128;
  const dim3 grid_dot((unsigned)((p.T * p.Hl * (p.D / 8) + NT - 1) / NT));
  LaunchInfo i0{d128 ? "attn_bwd_dot_d128" : "attn_bwd_dot_d64", 0.0, 2.0 * el + 4.0 * p.T * p.Hl};
  trace_begin(s);
  if (d128) hipLaunchKernelGGL(attn_bwd_dot_kernel<128>, grid_dot, dim3(NT), 0, s, a);
  else hipLaunchKernelGGL(attn_bwd_dot_kernel<64>, grid_dot, dim3(NT), 0, s, a);
  trace_end(s, i0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const double f = attention_fwd_flops(p);   // 2 products per allowed pair
  const dim3 grid((unsigned)((int64_t)a.nb * a.B * a.Hl));
  // dK, dV: S, dP, dV, dK (4 products); dQ: S^T, dP^T, dQ (3 products)
  LaunchInfo i1{d128 ? "attn_bwd_dkdv_d128" : "attn_bwd_dkdv_d64", 2.0 * f, 3.0 * el + 4.0 * 2 * p.T * p.Hl + 2.0 * el};
  trace_begin(s);
  if (d128) hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, grid, dim3(NT), 0, s, a);
  else hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, grid, dim3(NT), 0, s, a);
  trace_end(s, i1);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  LaunchInfo i2{d128 ? "attn_bwd_dq_d128" : "attn_bwd_dq_d64", 1.5 * f, 3.0 * el + 4.0 * 2 * p.T * p.Hl + el};
  trace_begin(s);
  if (d128) hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, grid, dim3(NT), 0, s, a);
  else hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, grid, dim3(NT), 0, s, a);
  trace_end(s, i2);
  return hipGetLastError();
}

}  // namespace tps
