// Core attention on one rank's local heads: for every head h and sequence b,
// O = softmax(Q K^T / sqrt(D) + M) V with M the causal mask (or none), bf16
// operands, fp32 scores and softmax, computed in one pass over the keys with a
// running maximum and sum (the exact IO-aware formulation: the T x T score
// matrix never reaches HBM).
//
// Forward kernel.  A workgroup owns 128 queries of one (sequence, head); each
// of its 4 waves owns 32 of them.  Keys and values stream through LDS in blocks
// of 64, double-buffered and copied HBM -> LDS directly (buffer loads with the
// LDS flag; no register staging).  Per block a wave computes
// the transposed scores S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so that
// each lane holds 32 scores of ONE query (its column) and the softmax
// statistics (running max m, running sum l) are per-lane scalars; the two lanes
// that share a query (lane and lane ^ 32) combine their maxima with one swap.
// The probabilities then feed O^T += V^T P^T straight from registers: the
// MFMA's k index (keys) is a summation index, so the keys are fed in the order
// the score accumulators hold them (per lane half: 4 keys, skip 4, 4 keys) and
// the V^T operand is read from LDS with transposing reads in that same order.
// The O^T accumulator again has one query per lane, so the rescale by
// exp(m_old - m_new) is a per-lane multiply.  K runs one block ahead of V:
// while a block's probabilities are formed, the next block's scores are
// computed, so the vector work sits between MFMAs of the same wave.  The
// running maximum a lane's probabilities are taken against moves only when a
// block exceeds it by more than 2^8 (RESCALE_LOG2), so the rescale is rare.
#include "attention.h"

#include <cmath>
#include <type_traits>

#include "lds_dma.h"

namespace tps {
namespace {

constexpr int AW = 4;            // waves per workgroup
constexpr int QW = 32;           // queries per wave
constexpr int BQ = AW * QW;      // queries per workgroup
constexpr int BKEYS = 64;        // keys per LDS block
constexpr int NT = AW * 64;      // threads per workgroup
static_assert(NT == kAttnThreads, "the launch-size check assumes kAttnThreads work-items per workgroup");

template <int D>
struct Shape {
  static constexpr int CH = D / 8;                      // 16-byte chunks per K/V row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int BLOCK_BYTES = BKEYS * ROW_BYTES;  // one K (or V) block
  static constexpr int KS = D / 16;                     // 16-wide d slices of a score product
  static constexpr int DT = D / 32;                     // 32-row d tiles of O^T
  static_assert(BLOCK_BYTES % (1024 * AW) == 0, "whole 1 KiB copies per wave per block");
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

// The Q / dO blocks of the dK/dV kernel use a second permutation, made for its
// transposing reads of 16 x 16 operand blocks as well as its row reads (16
// lanes read chunk c of 16 consecutive rows: f(r) takes 16 distinct values on
// 16 aligned rows).  A transposing read's 16-lane group covers 4 rows x 32
// bytes (chunks 2j, 2j + 1), group g rows 4g .. 4g + 3, and the LDS serves
// groups 0 and 2 together, 1 and 3 together (measured: a permutation that kept
// each run of 8 rows apart but not rows 0-3 from 8-11 cost 13 M bank-conflict
// cycles per 175B-shaped launch; this one none), so f(r) / 2 must differ on
// rows {0-3, 8-11} and on {4-7, 12-15} -- and, for D = 64 (two 128-byte rows
// per 256-byte bank sweep), among the rows of one parity in those sets.
//  D = 128: f(r) = 2 ((r mod 4) + 4 x) + (r / 8 mod 2);
//  D = 64:  f(r) = 2 ((r / 2 mod 2) + 2 x) + (r / 8 mod 2),  x = (r / 4 xor r / 8) mod 2.
template <int D>
__device__ __forceinline__ int qd_slot(int c, int r) {
  const int x = ((r >> 2) ^ (r >> 3)) & 1;
  return D == 128 ? c ^ (2 * ((r & 3) + 4 * x) + ((r >> 3) & 1)) : c ^ (2 * (((r >> 1) & 1) + 2 * x) + ((r >> 3) & 1));
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_bf16: A lane l holds row l % 16, k = 8 (l / 16) + 0..7;
// B lane l holds column l % 16, the same k; D lane l holds column l % 16, rows
// 4 (l / 16) + 0..3.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The value held by lane ^ 32 (xhalf = (lane ^ 32) * 4).
__device__ __forceinline__ float other_half(float v, int xhalf) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(xhalf, __float_as_int(v)));
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

// Per-lane LDS byte offsets of one wave's operand reads inside a K (or V)
// block.  The swizzle depends only on the low four bits of a row, which the
// row steps of the loops (32 keys for K, 16 keys for V) leave unchanged, so the
// steps, the buffer and the K/V half are compile-time offsets on top of these.
template <int D>
struct KvReadOffsets {
  int k[Shape<D>::KS];                       // K rows l32 (+ 32 t), 16-wide d slice s
  int va[Shape<D>::DT], vb[Shape<D>::DT];    // V transposing reads, d tile t: rows tr_r, tr_r + 8 (+ 16 s)
  __device__ __forceinline__ void init(int l32, int hh, int tr_r, int tr_c) {
#pragma unroll
    for (int s = 0; s < Shape<D>::KS; ++s) k[s] = l32 * Shape<D>::ROW_BYTES + kv_slot<D>(2 * s + hh, l32) * 16;
#pragma unroll
    for (int t = 0; t < Shape<D>::DT; ++t) {
      const int col = 32 * t + tr_c;
      va[t] = tr_r * Shape<D>::ROW_BYTES + kv_slot<D>(col >> 3, tr_r) * 16 + (col & 7) * 2;
      vb[t] = (tr_r + 8) * Shape<D>::ROW_BYTES + kv_slot<D>(col >> 3, tr_r + 8) * 16 + (col & 7) * 2;
    }
  }
};

// Copies of 64-row blocks of a [rows x D] slice (row stride ld elements)
// straight into LDS in the kv_slot layout: each wave moves NI KiB of a block,
// lane i of copy c landing at byte 1024 (wave NI + c) + 16 i, which is chunk
// slot s of row r; it fetches the chunk that the swizzle puts there.  Rows at
// or past `rows_left` read as zero through the buffer range check.
template <int D, bool QD = false, int ROWS = BKEYS>
struct BlockCopier {
  static constexpr int NI = ROWS * Shape<D>::ROW_BYTES / 1024 / AW;
  static_assert(NI * 1024 * AW == ROWS * Shape<D>::ROW_BYTES, "whole 1 KiB copies per wave per block");
  int off[NI];
  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = (wave * NI + i) * 64 + lane;
      const int r = q / Shape<D>::CH, sl = q % Shape<D>::CH;
      off[i] = r * (int)(ld * 2) + (QD ? qd_slot<D>(sl, r) : kv_slot<D>(sl, r)) * 16;
    }
  }
  // Block starting at `first` (row 0 of the copy); `rows_left` rows from there are data.
  __device__ __forceinline__ void issue(const bf16* first, int64_t ld, int rows_left, unsigned lds, int wave) const {
    const i32x4 rs = make_rsrc(first, rows_left > 0 ? ((int64_t)(rows_left - 1) * ld + D) * 2 : 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) lds_dma16(rs, off[i], lds + (wave * NI + i) * 1024);
  }
};

// Lazy rescaling: a lane's reference maximum m moves only when a block's
// maximum exceeds it by more than this many powers of two, so probabilities
// are at most 2^8 (exact in fp32, and bf16 keeps fp32's exponent range) and the
// O accumulators are rescaled only on the rare blocks where m moves.
constexpr float RESCALE_LOG2 = 8.0f;

template <int D>
__global__ void __launch_bounds__(NT, 2) attn_fwd_kernel(FwdArgs a) {
  using SH = Shape<D>;
  constexpr int BUF = 2 * SH::BLOCK_BYTES;  // one buffer: a K block, then a V block
  constexpr int EPS = 32 / SH::KS;           // score elements converted per 16-wide d slice
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // Keys at or past `lim` are masked for this lane's query.
  const int lim = a.causal ? min(a.S, qi + 1) : a.S;
  const int xhalf = (lane ^ 32) << 2;      // ds_bpermute address of the lane sharing this query

  BlockCopier<D> cp;
  cp.init(ld, wave, lane);
  const unsigned lds0 = lds_address(smem);
  auto issue_k = [&](int j, int buf) {
    cp.issue(kbase + (int64_t)j * BKEYS * ld, ld, a.S - j * BKEYS, lds0 + buf * BUF, wave);
  };
  auto issue_v = [&](int j, int buf) {
    cp.issue(vbase + (int64_t)j * BKEYS * ld, ld, a.S - j * BKEYS, lds0 + buf * BUF + SH::BLOCK_BYTES, wave);
  };
  // K runs one block ahead of V: block j's K is in buffer j % 2 until its
  // scores are computed (during block j - 1), its V until block j is done.
  issue_k(0, 0);
  issue_v(0, 0);
  if (nkb > 1) issue_k(1, 1);

  // Q operand (k = d, column = query), resident for the whole key loop.
  bf16x8 qf[SH::KS];
#pragma unroll
  for (int s = 0; s < SH::KS; ++s)
    qf[s] = qvalid ? *(const bf16x8*)(qbase + (int64_t)qi * ld + 16 * s + 8 * hh) : bf16x8{};

  // Transposing-read coordinates of this lane (16-lane group g = lane / 16:
  // lane half g / 2, column half g % 2).
  const int g16 = lane >> 4, i16 = lane & 15;
  KvReadOffsets<D> ro;
  ro.init(l32, hh, 4 * (g16 >> 1) + (i16 >> 2), 16 * (g16 & 1) + 4 * (i16 & 3));

  f32x16 oacc[SH::DT];
#pragma unroll
  for (int t = 0; t < SH::DT; ++t) oacc[t] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.0f;

  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  // S^T[key][query] of one block (keys 32 t + (0..31) in sc[t]) from the K
  // block at Ks; the operands of slice s + 1 are read while slice s runs.
  auto kfrag = [&](const char* Ks, int s, int t) {
    return *(const bf16x8*)(Ks + ro.k[s] + t * 32 * SH::ROW_BYTES);
  };
  f32x16 scA[2] = {f32x16{}, f32x16{}}, scB[2];
  {
    bf16x8 kf[2][2];
    kf[0][0] = kfrag(smem, 0, 0);
    kf[0][1] = kfrag(smem, 0, 1);
#pragma unroll
    for (int s = 0; s < SH::KS; ++s) {
      if (s + 1 < SH::KS) {
        kf[(s + 1) & 1][0] = kfrag(smem, s + 1, 0);
        kf[(s + 1) & 1][1] = kfrag(smem, s + 1, 1);
      }
      scA[0] = mfma(kf[s & 1][0], qf[s], scA[0]);
      scA[1] = mfma(kf[s & 1][1], qf[s], scA[1]);
    }
  }
  __syncthreads();  // block 0's K buffer is free for block 2

  // Key block j (BI = j % 2, a constant, so every LDS address is a per-lane
  // base plus an immediate): its scores are in sc; the next block's scores are
  // computed into sn while this block's probabilities are formed, so the
  // matrix cores and the vector ALU work side by side.
  auto block = [&](int j, auto bic, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr int BI = decltype(bic)::value;
    const int k0 = j * BKEYS;
    // Mask (only blocks that reach past the sequence end or this wave's first
    // query) and this lane's block maximum on the raw scores (the scale is positive).
    if ((k0 + BKEYS > a.S) || (a.causal && k0 + BKEYS - 1 > wq0)) {
      const int x = lim - k0 - 4 * hh;  // accumulator element (t, v) is key k0 + 4 hh + c(t, v)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int c = 32 * t + 8 * (v >> 2) + (v & 3);
          sc[t][v] = c >= x ? -INFINITY : sc[t][v];
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, sc[t][v]);
    mloc = fmaxf(mloc, other_half(mloc, xhalf));
    const float mblk = mloc * a.scale_log2;  // finite on block 0: key 0 is allowed for every query
    if (__ballot(mblk > m_ref + RESCALE_LOG2) != 0) {
      const float m_new = mblk > m_ref + RESCALE_LOG2 ? mblk : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < SH::DT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[t][v] *= alpha;
      m_ref = m_new;
    }

    // Copies: block j + 2's K into this K buffer (its scores were computed
    // before the last barrier), block j + 1's V into the other V buffer.
    if (j + 2 < nkb) issue_k(j + 2, BI);
    if (j + 1 < nkb) issue_v(j + 1, BI ^ 1);

    // Block j + 1's scores (garbage past the last block, then unused), slice
    // by slice, each slice followed by its share of block j's probabilities
    // p = 2^(s * log2(e)/sqrt(D) - m) (one FMA and an exp2), packed to bf16 as
    // the B operand of O^T += V^T P^T: k slot m of 16-key slice q and lane half
    // hh is key 16 q + 8 (m / 4) + 4 hh + m % 4, i.e. score element 8 q + m.
    const char* Kn = smem + (BI ^ 1) * BUF;
    const char* Vs = smem + BI * BUF + SH::BLOCK_BYTES;
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    bf16x8 pf[4];
    float ps0 = 0.0f, ps1 = 0.0f;
    bf16x8 kf[2][2];
    kf[0][0] = kfrag(Kn, 0, 0);
    kf[0][1] = kfrag(Kn, 0, 1);
#pragma unroll
    for (int s = 0; s < SH::KS; ++s) {
      if (s + 1 < SH::KS) {
        kf[(s + 1) & 1][0] = kfrag(Kn, s + 1, 0);
        kf[(s + 1) & 1][1] = kfrag(Kn, s + 1, 1);
      }
      sn[0] = mfma(kf[s & 1][0], qf[s], sn[0]);
      sn[1] = mfma(kf[s & 1][1], qf[s], sn[1]);
#pragma unroll
      for (int e = EPS * s; e < EPS * (s + 1); e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e >> 4][e & 15], a.scale_log2, -m_ref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e >> 4][(e + 1) & 15], a.scale_log2, -m_ref));
        pf[e >> 3][e & 7] = (bf16)p0;
        pf[e >> 3][(e + 1) & 7] = (bf16)p1;
        ps0 += p0;
        ps1 += p1;
      }
    }
    l_run += ps0 + ps1;

    // O^T[d][query] += V^T P^T; V^T read with the same key order, one operand
    // ahead of the MFMA that uses it.
    auto vfrag = [&](int s, int t) {
      const bf16x4 lo = read_tr(Vs + ro.va[t] + 16 * s * SH::ROW_BYTES);
      const bf16x4 hi = read_tr(Vs + ro.vb[t] + 16 * s * SH::ROW_BYTES);
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

    // This wave's copies have landed and every wave is done with the buffers
    // the next block's copies overwrite.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
  };
  for (int j = 0; j < nkb; j += 2) {
    block(j, std::integral_constant<int, 0>{}, scA, scB);
    if (j + 1 < nkb) block(j + 1, std::integral_constant<int, 1>{}, scB, scA);
  }

  const float l_tot = l_run + other_half(l_run, xhalf);
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
      a.lse[(int64_t)h * a.T + row0 + qi] = (m_ref + __log2f(l_tot)) * 0.6931471805599453f;
  }
}

// ---------------------------------------------------------------- backward
//
// With P the forward's probabilities (recomputed from the saved log-sum-exp),
// dP = dO V^T and Dt = rowsum(dO * O) = rowsum(P * dP):
//   dV = P^T dO,  dS = P * (dP - Dt),  dK = dS^T Q / sqrt(D),  dQ = dS K / sqrt(D).
// Two kernels, no atomics (bitwise reproducible), dQ first:
//  * attn_bwd_dq (below) also forms Dt for its queries from the dO rows it
//    holds and the matching O rows, and writes it for attn_bwd_dkdv;
//  * attn_bwd_dkdv: a workgroup owns 64 keys (16 per wave, one per lane
//    column of 16 x 16 x 32 MFMAs, two workgroups per CU); K and V of its keys
//    stay in registers; queries (Q and dO rows) are copied HBM -> LDS directly
//    in double-buffered blocks of 64.  Scores are computed as S[query][key] so
//    each lane holds one key's column, and P and dS feed dV^T += dO^T P and
//    dK^T += Q^T dS from registers (queries in the accumulator order, dO^T and
//    Q^T read from LDS with transposing reads in that order);
//  * attn_bwd_dq, its mirror: a workgroup owns 64 queries (16 per wave, one per
//    lane column, two workgroups per CU) whose Q and dO stay in registers; keys
//    and values are copied HBM -> LDS directly in double-buffered blocks of 64;
//    S^T and dP^T = V dO^T give dS^T, which feeds dQ^T += K^T dS^T.

struct BwdArgs {
  const bf16* qkv;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  float* dt;        // [Hl x T]
  bf16* dqkv;
  int64_t T;
  int S, Hl, B, causal;
  float scale_log2;           // log2(e) / sqrt(D)
  float scale;                // 1 / sqrt(D)
};

constexpr float LOG2E = 1.4426950408889634f;

// dK/dV with 16 keys per wave on 16 x 16 x 32 MFMAs.  A workgroup owns 64 keys
// (4 waves x 16, one key per lane column); with K, V, dK, dV, S and dP of 16
// keys a wave needs fewer than 256 registers, so two workgroups share each CU
// and a SIMD runs two waves of different workgroups, which do not wait at each
// other's barriers and whose MFMAs cover each other's softmax arithmetic.  Per 64-query block (Q and dO copied HBM ->
// LDS directly, double-buffered, in the qd_slot layout):
//  * S[q][key] and dP[q][key] for 4 blocks of 16 queries (A: Q / dO rows read
//    from LDS, B: this wave's K / V in registers, k = d);
//  * P and dS in registers, packed as the B operand of dV^T += dO^T P and
//    dK^T += Q^T dS over 32-query k blocks: k slot 8 g + e of lane half g is
//    query 4 g + (e mod 4) + 16 (e / 4) of the k block, the order the score
//    accumulators hold them, and dO^T / Q^T are read with transposing reads of
//    rows 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3 in that same order.
template <int D>
__global__ void __launch_bounds__(NT, 2) attn_bwd_dkdv_kernel(BwdArgs a) {
  using SH = Shape<D>;
  constexpr int QB = 64;                     // queries per LDS block
  constexpr int KW = 16;                     // keys per wave
  constexpr int BKW = AW * KW;               // keys per workgroup
  constexpr int BUF = 2 * SH::BLOCK_BYTES;   // one buffer: a Q block, then a dO block
  constexpr int NS = D / 32;                 // 32-wide d slices: k of S and dP
  constexpr int NDB = D / 16;                // 16-row d blocks of dK^T and dV^T
  constexpr int RB = SH::ROW_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF];
  __shared__ __attribute__((aligned(16))) float stat[2][2][QB];  // [buffer][lse * log2(e), Dt]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int bh = a.B * a.Hl;
  const int kb = (int)(blockIdx.x / bh);           // causal: low key blocks have the most queries
  const int b = (int)(blockIdx.x % bh) / a.Hl, h = (int)(blockIdx.x % bh) % a.Hl;
  const int64_t ld = 3LL * a.Hl * D;
  const int64_t row0 = (int64_t)b * a.S;
  const bf16* qbase = a.qkv + row0 * ld + (int64_t)h * D;
  const bf16* kbase = qbase + (int64_t)a.Hl * D;
  const bf16* vbase = qbase + 2LL * a.Hl * D;
  const int64_t ldo = (int64_t)a.Hl * D;
  const bf16* dobase = a.dout + row0 * ldo + (int64_t)h * D;
  const int kw0 = kb * BKW + wave * KW;            // first key of this wave
  const int kj = kw0 + l16;                        // this lane's key
  const bool kvalid = kj < a.S;
  const int qstart = a.causal ? kb * BKW : 0;      // earlier queries see none of these keys
  const int nqblk = (a.S - qstart + QB - 1) / QB;

  BlockCopier<D, true> cq, co;
  cq.init(ld, wave, lane);
  co.init(ldo, wave, lane);
  const unsigned lds0 = lds_address(smem);
  auto issue = [&](int j, int buf) {
    const int q0 = qstart + j * QB;
    cq.issue(qbase + (int64_t)q0 * ld, ld, a.S - q0, lds0 + buf * BUF, wave);
    co.issue(dobase + (int64_t)q0 * ldo, ldo, a.S - q0, lds0 + buf * BUF + SH::BLOCK_BYTES, wave);
  };
  // The block's per-query statistics go through wave 0's registers (2 x 64 floats).
  float st_l2 = 0.0f, st_dt = 0.0f;
  auto load_stats = [&](int q0) {
    if (wave == 0) {
      const int q = q0 + lane;
      st_l2 = q < a.S ? a.lse[(int64_t)h * a.T + row0 + q] * LOG2E : INFINITY;
      st_dt = q < a.S ? a.dt[(int64_t)h * a.T + row0 + q] : 0.0f;
    }
  };
  auto store_stats = [&](int buf) {
    if (wave == 0) {
      stat[buf][0][lane] = st_l2;
      stat[buf][1][lane] = st_dt;
    }
  };
  issue(0, 0);
  load_stats(qstart);

  // K and V of this lane's key as the B operand of S and dP: d = 32 s + 8 g + 0..7.
  bf16x8 kf[NS], vf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = kvalid ? *(const bf16x8*)(kbase + (int64_t)kj * ld + 32 * s + 8 * g) : bf16x8{};
    vf[s] = kvalid ? *(const bf16x8*)(vbase + (int64_t)kj * ld + 32 * s + 8 * g) : bf16x8{};
  }
  // Row reads: query 16 t + l16, chunk 4 s + g (the swizzle depends on the row
  // mod 16 only, so t is an immediate).  Transposing reads of d block db: row
  // 4 g + l16 / 4 (+ 16, + 32 kq: immediates), column 16 db + 4 (l16 mod 4).
  int rowo[NS], tro[NDB];
#pragma unroll
  for (int s = 0; s < NS; ++s) rowo[s] = l16 * RB + qd_slot<D>(4 * s + g, l16) * 16;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int r = 4 * g + (l16 >> 2);
    tro[db] = r * RB + qd_slot<D>(2 * db + ((l16 >> 1) & 1), r) * 16 + (l16 & 1) * 8;
  }

  f32x4 dk[NDB], dv[NDB];
#pragma unroll
  for (int t = 0; t < NDB; ++t) { dk[t] = f32x4{}; dv[t] = f32x4{}; }

  store_stats(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  // Query block j from LDS buffer BI = j % 2 (a constant, so every LDS address
  // is a per-lane base plus an immediate) while block j + 1 is copied into the
  // other buffer.
  auto block = [&](int j, auto bic) {
    constexpr int BI = decltype(bic)::value;
    const int q0 = qstart + j * QB;
    if (j + 1 < nqblk) {
      issue(j + 1, BI ^ 1);
      load_stats(q0 + QB);
    }
    const char* Qs = smem + BI * BUF;
    const char* Gs = Qs + SH::BLOCK_BYTES;

    // S and dP of queries 16 t + (0..15) of the block, t = n / NS, d slice
    // s = n % NS; the Q and dO operands are read RD steps ahead.
    constexpr int RD = 3, NSTEP = 4 * NS;
    f32x4 sc[4], dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) { sc[t] = f32x4{}; dp[t] = f32x4{}; }
    bf16x8 qr[RD + 1], gr[RD + 1];
    auto rows = [&](int n) {
      const int o = rowo[n % NS] + (n / NS) * 16 * RB;
      qr[n % (RD + 1)] = *(const bf16x8*)(Qs + o);
      gr[n % (RD + 1)] = *(const bf16x8*)(Gs + o);
    };
#pragma unroll
    for (int n = 0; n < RD; ++n) rows(n);
#pragma unroll
    for (int n = 0; n < NSTEP; ++n) {
      if (n + RD < NSTEP) rows(n + RD);
      sc[n / NS] = mfma16(qr[n % (RD + 1)], kf[n % NS], sc[n / NS]);
      dp[n / NS] = mfma16(gr[n % (RD + 1)], vf[n % NS], dp[n / NS]);
    }
    // Keep the operand reads RD steps ahead.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RD, 0);
#pragma unroll
    for (int n = 0; n < NSTEP; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (n + RD < NSTEP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // Causal mask, only where some query of the block precedes one of this
    // wave's keys: element (t, r) is query q0 + 16 t + 4 g + r.
    if (a.causal && q0 < kw0 + KW - 1) {
      const int x = kj - q0 - 4 * g;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[t][r] = 16 * t + r < x ? -INFINITY : sc[t][r];
    }
    // dO^T and Q^T operands of 32-query k block kq, d block db.
    auto tr = [&](const char* base, int kq, int db) {
      const char* p = base + tro[db] + 32 * kq * RB;
      const bf16x4 lo = read_tr(p), hi = read_tr(p + 16 * RB);
      bf16x8 v;
      v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
      v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
      return v;
    };
    constexpr int NOP = 2 * NDB, VPD = 6;
    bf16x8 gv[VPD], qv[VPD];
    auto tr_pair = [&](int n) {
      gv[n % VPD] = tr(Gs, n / NDB, n % NDB);
      qv[n % VPD] = tr(Qs, n / NDB, n % NDB);
    };
#pragma unroll
    for (int n = 0; n < VPD; ++n) tr_pair(n);
    // P and dS of k block kq (score blocks t = 2 kq, 2 kq + 1).
    bf16x8 pf[2], sf[2];
    auto pds = [&](int kq, int u) {
      const int t = 2 * kq + u;
      const f32x4 l2 = *(const f32x4*)&stat[BI][0][16 * t + 4 * g];
      const f32x4 dd = *(const f32x4*)&stat[BI][1][16 * t + 4 * g];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][r], a.scale_log2, -l2[r]));
        pf[kq][4 * u + r] = (bf16)p;
        sf[kq][4 * u + r] = (bf16)(p * (dp[t][r] - dd[r]));
      }
    };
    pds(0, 0);
    pds(0, 1);
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int n = kq * NDB + db;
        dv[db] = mfma16(gv[n % VPD], pf[kq], dv[db]);
        dk[db] = mfma16(qv[n % VPD], sf[kq], dk[db]);
        if (n + VPD < NOP) tr_pair(n + VPD);
      }
      if (kq == 0) {
        pds(1, 0);
        pds(1, 1);
      }
    }
    if (j + 1 < nqblk) store_stats(BI ^ 1);
    // This wave's copies have landed and every wave is done with this buffer.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
  };
  for (int j = 0; j < nqblk; j += 2) {
    block(j, std::integral_constant<int, 0>{});
    if (j + 1 < nqblk) block(j + 1, std::integral_constant<int, 1>{});
  }

  if (kvalid) {
    bf16* krow = a.dqkv + (row0 + kj) * ld + (int64_t)a.Hl * D + (int64_t)h * D;
    bf16* vrow = krow + (int64_t)a.Hl * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x4 k4, v4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        k4[r] = (bf16)(dk[db][r] * a.scale);
        v4[r] = (bf16)dv[db][r];
      }
      *(bf16x4*)(krow + 16 * db + 4 * g) = k4;
      *(bf16x4*)(vrow + 16 * db + 4 * g) = v4;
    }
  }
}

// dQ with 16 queries per wave on 16 x 16 x 32 MFMAs, the mirror of the dK/dV
// kernel: a workgroup owns 64 queries (4 waves x 16, one query per lane column),
// whose Q and dO stay in registers; keys and values stream through LDS in
// double-buffered blocks of 64 (qd_slot layout: K is read both as rows and with
// transposing reads).  Per block:
//  * S^T[key][q] and dP^T[key][q] for 4 tiles of 16 keys (A: K / V rows from
//    LDS, B: this wave's Q / dO, k = d); a lane holds keys 16 t + 4 g + 0..3 of
//    its query, so the softmax statistics (lse, Dt) are per-lane constants;
//  * dS^T in registers as the B operand of dQ^T += K^T dS^T over 32-key k
//    blocks, in the accumulator order (k slot 8 g + e is key 4 g + (e mod 4) +
//    16 (e / 4) of the k block), K^T read with transposing reads in that order.
// Dt = rowsum(dO * O) for the workgroup's queries is formed here from the dO
// the lanes hold (32 of a row's d per lane, the 4 lanes of a query added in a
// fixed order) and written for the dK/dV kernel.  Workgroups of 64 queries let
// the longest causal rows (all keys) take less than a workgroup slot's mean load.
template <int D, int KB>
__global__ void __launch_bounds__(NT, 2) attn_bwd_dq_kernel(BwdArgs a) {
  using SH = Shape<D>;
  constexpr int QW16 = 16;                   // queries per wave
  constexpr int BQ16 = AW * QW16;            // queries per workgroup
  constexpr int KBYTES = KB * SH::ROW_BYTES; // one K (or V) block of KB keys
  constexpr int BUF = 2 * KBYTES;            // one buffer: a K block, then a V block
  constexpr int NTL = KB / 16;               // 16-key tiles per block
  constexpr int NKQ = KB / 32;               // 32-key k blocks per block
  constexpr int NS = D / 32;                 // 32-wide d slices: k of S^T and dP^T
  constexpr int NDB = D / 16;                // 16-row d blocks of dQ^T
  constexpr int RB = SH::ROW_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int bh = a.B * a.Hl;
  const int nqb = (a.S + BQ16 - 1) / BQ16;
  const int qb = nqb - 1 - (int)(blockIdx.x / bh);  // longest causal query blocks first
  const int b = (int)(blockIdx.x % bh) / a.Hl, h = (int)(blockIdx.x % bh) % a.Hl;
  const int64_t ld = 3LL * a.Hl * D;
  const int64_t row0 = (int64_t)b * a.S;
  const bf16* qbase = a.qkv + row0 * ld + (int64_t)h * D;
  const bf16* kbase = qbase + (int64_t)a.Hl * D;
  const bf16* vbase = qbase + 2LL * a.Hl * D;
  const int64_t ldo = (int64_t)a.Hl * D;
  const bf16* dobase = a.dout + row0 * ldo + (int64_t)h * D;
  const int q0 = qb * BQ16;
  const int wq0 = q0 + wave * QW16;                  // first query of this wave
  const int qi = wq0 + l16;                          // this lane's query
  const bool qvalid = qi < a.S;
  const int kend = a.causal ? min(a.S, q0 + BQ16) : a.S;
  const int nkb = (kend + KB - 1) / KB;
  const int lim = a.causal ? min(a.S, qi + 1) : a.S;  // keys at or past lim are masked

  BlockCopier<D, true, KB> cp;
  cp.init(ld, wave, lane);
  const unsigned lds0 = lds_address(smem);
  auto issue = [&](int j, int buf) {
    const int k0 = j * KB;
    cp.issue(kbase + (int64_t)k0 * ld, ld, a.S - k0, lds0 + buf * BUF, wave);
    cp.issue(vbase + (int64_t)k0 * ld, ld, a.S - k0, lds0 + buf * BUF + KBYTES, wave);
  };
  issue(0, 0);

  // Q and dO of this lane's query as the B operand of S^T and dP^T: d = 32 s + 8 g + 0..7.
  bf16x8 qf[NS], gf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = qvalid ? *(const bf16x8*)(qbase + (int64_t)qi * ld + 32 * s + 8 * g) : bf16x8{};
    gf[s] = qvalid ? *(const bf16x8*)(dobase + (int64_t)qi * ldo + 32 * s + 8 * g) : bf16x8{};
  }
  const float lse2 = qvalid ? a.lse[(int64_t)h * a.T + row0 + qi] * LOG2E : INFINITY;
  // Dt = rowsum(dO * O): this lane's 32 products, then the 4 lanes of the query
  // (l16 + 16 g) added pairwise; fp32 addition commutes, so all four hold the same value.
  float dti = 0.0f;
  {
    const bf16* orow = a.o + (row0 + qi) * ldo + (int64_t)h * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 ov = qvalid ? *(const bf16x8*)(orow + 32 * s) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) dti += (float)gf[s][e] * (float)ov[e];
    }
    dti += __shfl_xor(dti, 16);
    dti += __shfl_xor(dti, 32);
    if (qvalid && g == 0) a.dt[(int64_t)h * a.T + row0 + qi] = dti;
  }
  // Row reads: key 16 t + l16, chunk 4 s + g.  Transposing reads of d block db:
  // key row 4 g + l16 / 4 (+ 16, + 32 kq: immediates), column 16 db + 4 (l16 mod 4).
  int rowo[NS], tro[NDB];
#pragma unroll
  for (int s = 0; s < NS; ++s) rowo[s] = l16 * RB + qd_slot<D>(4 * s + g, l16) * 16;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int r = 4 * g + (l16 >> 2);
    tro[db] = r * RB + qd_slot<D>(2 * db + ((l16 >> 1) & 1), r) * 16 + (l16 & 1) * 8;
  }

  f32x4 dq[NDB];
#pragma unroll
  for (int t = 0; t < NDB; ++t) dq[t] = f32x4{};

  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  auto block = [&](int j, auto bic) {
    constexpr int BI = decltype(bic)::value;
    const int k0 = j * KB;
    if (j + 1 < nkb) issue(j + 1, BI ^ 1);
    const char* Ks = smem + BI * BUF;
    const char* Vs = Ks + KBYTES;

    // S^T and dP^T of keys 16 t + (0..15) of the block, t = n / NS, d slice
    // s = n % NS; the K and V operands are read RD steps ahead.
    constexpr int RD = 3, NSTEP = NTL * NS;
    f32x4 sc[NTL], dp[NTL];
#pragma unroll
    for (int t = 0; t < NTL; ++t) { sc[t] = f32x4{}; dp[t] = f32x4{}; }
    bf16x8 kr[RD + 1], vr[RD + 1];
    auto rows = [&](int n) {
      const int o = rowo[n % NS] + (n / NS) * 16 * RB;
      kr[n % (RD + 1)] = *(const bf16x8*)(Ks + o);
      vr[n % (RD + 1)] = *(const bf16x8*)(Vs + o);
    };
#pragma unroll
    for (int n = 0; n < RD; ++n) rows(n);
#pragma unroll
    for (int n = 0; n < NSTEP; ++n) {
      if (n + RD < NSTEP) rows(n + RD);
      sc[n / NS] = mfma16(kr[n % (RD + 1)], qf[n % NS], sc[n / NS]);
      dp[n / NS] = mfma16(vr[n % (RD + 1)], gf[n % NS], dp[n / NS]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RD, 0);
#pragma unroll
    for (int n = 0; n < NSTEP; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (n + RD < NSTEP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // Mask (blocks reaching past the sequence end or this wave's first query):
    // element (t, r) is key k0 + 16 t + 4 g + r.
    if (k0 + KB > a.S || (a.causal && k0 + KB - 1 > wq0)) {
      const int x = lim - k0 - 4 * g;
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[t][r] = 16 * t + r < x ? sc[t][r] : -INFINITY;
    }
    // K^T operand of 32-key k block kq, d block db.
    auto tr = [&](int kq, int db) {
      const char* p = Ks + tro[db] + 32 * kq * RB;
      const bf16x4 lo = read_tr(p), hi = read_tr(p + 16 * RB);
      bf16x8 v;
      v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
      v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
      return v;
    };
    constexpr int NOP = NKQ * NDB, VPD = 4;
    bf16x8 kv[VPD];
#pragma unroll
    for (int n = 0; n < VPD; ++n) kv[n] = tr(n / NDB, n % NDB);
    // dS^T of k block kq (score tiles t = 2 kq, 2 kq + 1).
    bf16x8 sf[NKQ];
    auto pds = [&](int kq) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 2 * kq + u;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][r], a.scale_log2, -lse2));
          sf[kq][4 * u + r] = (bf16)(p * (dp[t][r] - dti));
        }
    };
    pds(0);
#pragma unroll
    for (int kq = 0; kq < NKQ; ++kq) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int n = kq * NDB + db;
        dq[db] = mfma16(kv[n % VPD], sf[kq], dq[db]);
        if (n + VPD < NOP) kv[n % VPD] = tr((n + VPD) / NDB, (n + VPD) % NDB);
      }
      if (kq + 1 < NKQ) pds(kq + 1);
    }
    // This wave's copies have landed and every wave is done with this buffer.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
  };
  for (int j = 0; j < nkb; j += 2) {
    block(j, std::integral_constant<int, 0>{});
    if (j + 1 < nkb) block(j + 1, std::integral_constant<int, 1>{});
  }

  if (qvalid) {
    bf16* qrow = a.dqkv + (row0 + qi) * ld + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x4 q4;
#pragma unroll
      for (int r = 0; r < 4; ++r) q4[r] = (bf16)(dq[db][r] * a.scale);
      *(bf16x4*)(qrow + 16 * db + 4 * g) = q4;
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
  a.causal = p.causal ? 1 : 0;
  a.scale = (float)(1.0 / std::sqrt((double)p.D));
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p.D));
  const double el = 2.0 * p.T * p.Hl * p.D;   // bytes of one [T x Hl*D] bf16 tensor
  const bool d128 = p.D == 128;
  const double f = attention_fwd_flops(p);   // 2 products per allowed pair
  // dQ: S^T, dP^T, dQ (3 products), and Dt for dK/dV (reads O as well);
  // dK, dV: S, dP, dV, dK (4 products)
  LaunchInfo i2{d128 ? "attn_bwd_dq_d128" : "attn_bwd_dq_d64", 1.5 * f,
                4.0 * el + 4.0 * p.T * p.Hl + el};
  trace_begin(s);
  const dim3 grid64q((unsigned)((int64_t)((p.S + 63) / 64) * a.B * a.Hl));  // 64 queries per workgroup
  if (d128) hipLaunchKernelGGL((attn_bwd_dq_kernel<128, 64>), grid64q, dim3(NT), 0, s, a);
  else hipLaunchKernelGGL((attn_bwd_dq_kernel<64, 64>), grid64q, dim3(NT), 0, s, a);
  trace_end(s, i2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  LaunchInfo i1{d128 ? "attn_bwd_dkdv_d128" : "attn_bwd_dkdv_d64", 2.0 * f, 3.0 * el + 4.0 * 2 * p.T * p.Hl + 2.0 * el};
  trace_begin(s);
  const dim3 grid64((unsigned)((int64_t)((p.S + 63) / 64) * a.B * a.Hl));  // 64 keys per workgroup
  if (d128) hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, grid64, dim3(NT), 0, s, a);
  else hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, grid64, dim3(NT), 0, s, a);
  trace_end(s, i1);
  return hipGetLastError();
}

}  // namespace tps
