// 16-bit (bf16 or fp16) GEMM with fused epilogues on the gfx950 matrix cores.
//
// C[M x N] = op(A)[M x K] * op(B)[K x N], fp32 accumulation in
// v_mfma_f32_32x32x16_bf16 (or its fp16 twin), one epilogue applied to the accumulators in
// registers before the only store (bias, bias + exact-erf GeLU with the
// pre-activation saved, GeLU' for the backward, or fp32 store / accumulate).
//
// Data path.  A workgroup owns a BM x BN tile of C.  The K loop walks K in steps
// of 32 through a ring of up to five LDS stages: each step's A and B panels are
// copied HBM -> LDS by buffer_load_dwordx4 ... lds (no register staging; rows
// and columns outside the matrix read as zero through the buffer range check)
// several steps ahead of the step the matrix cores work on.  Consumer waves
// read their MFMA operands from LDS and keep their fp32 accumulators in
// registers for the whole K loop.
//
// Wave organisation.  A copy instruction holds up its wave's instruction issue
// for tens of cycles, so a SIMD needs a second wave to keep the matrix pipe fed:
//  * "split" kernels (tiles up to 256 x 192): 8 consumer waves (2 per SIMD) and
//    4 producer waves that only issue the copies;
//  * "shared" kernels (256 x 384, 384 x 256, 192 x 384, 256 x 256): 8 waves,
//    each a consumer of a 128 x 96 (96 x 128, 96 x 96, 128 x 64) sub-tile; all
//    8 also issue the copies, except in 192 x 384, whose 36 KiB per step do not split
//    eight ways: there waves 0-3, one per SIMD, issue 9 copies each (six
//    copying waves would put 12 copies per step on two SIMDs and 6 on the
//    others, and the per-step barrier waits for the busiest).  The biggest tile moves 29% fewer bytes per FLOP from L2 and
//    reads 31% fewer operand bytes from LDS than 256 x 192, which matters
//    because the chip runs at its power limit and data movement lowers the
//    clock; 192 x 384 sits in between and fills whole waves of 256 tiles
//    where the others leave a partial wave (the 12288 x 4608 and 1536 x 12288
//    weight gradients).
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
// of C; the epilogue stages them through LDS and writes whole 16-byte runs of
// rows (and reads GeLU's Z the same way).
//
// Bias gradients.  A weight gradient dW = X^T dY can also return the column
// sums of its B operand dY (db = sum_t dY) from the B panels already in LDS
// (BColSum), so the gradient is not read from HBM a second time.
//
// Edges.  M, N and K may be ragged against the tile (T is arbitrary); loads
// outside the matrix read zero and stores outside it are skipped.  Feature
// dimensions are multiples of 8, so a 16-byte vector is entirely inside or
// entirely outside.
#include "gelu.h"
#include "gemm.h"
#include "lds_dma.h"

#include <algorithm>
#include <string>
#include <type_traits>

namespace tps {
namespace {

constexpr int KT = 32;        // K step per LDS stage

// The two 16-bit element types: operand vectors and the matching MFMA.
template <typename E> struct Vec;
template <> struct Vec<bf16> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  static constexpr const char* name = "bf16";
};
template <> struct Vec<f16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static constexpr const char* name = "f16";
};
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin,
// so consecutive ids are remapped to one XCD's contiguous range of logical
// tiles; logical tiles are ordered in groups of group_m tile rows so that an
// XCD's workgroups share A and B panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = bid & 7;
  const int local = bid >> 3;
  const int base = total >> 3;
  const int rem = total & 7;
  const int logical = xcd * base + (xcd < rem ? xcd : rem) + local;
  const int per_group = group_m * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * group_m;
  const int gsize = min(tiles_m - first_m, group_m);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

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


// Kernel shape: tile, waves and their roles, LDS ring.  NSHCOPY_ (shared
// kernels only): how many of the 8 waves issue the copies (waves 0 .. NSHCOPY_-1;
// a workgroup's waves go to the four SIMDs in turn), when a K step's 1 KiB
// copies do not divide evenly over all 8.
template <int BM_, int BN_, int NPROD_, int CM_, int NSHCOPY_ = 8>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int NCONS = 8, NPROD = NPROD_, NW = NCONS + NPROD, NT = 64 * NW;
  static constexpr int CM = CM_, CN = NCONS / CM_;
  static constexpr int WM = BM / CM, WN = BN / CN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_BYTES = BM * KT * 2, B_BYTES = BN * KT * 2, STAGE = A_BYTES + B_BYTES;
  static constexpr int NSTAGE = (163840 / STAGE) < 5 ? (163840 / STAGE) : 5;  // <= 160 KiB of LDS
  static constexpr int PREF = NSTAGE - 1;       // K steps in flight ahead of the one computed
  static constexpr int NCOPY = NPROD > 0 ? NPROD : NSHCOPY_;  // waves that issue the copies
  static constexpr int A_INS = A_BYTES / 1024 / NCOPY, B_INS = B_BYTES / 1024 / NCOPY;
  static constexpr int NVM = A_INS + B_INS;    // 1 KiB copies per copying wave per step
  static constexpr int WAVES_PER_EU = (NW + 3) / 4;
  static constexpr bool DBUF = NPROD > 0;       // double-buffered operands (register budget)
  // Column sums of B ride along (BColSum) on the tiles whose consumers have
  // registers to spare; the two biggest tiles are at the 256-register limit.
  static constexpr bool CSUM = BM * BN < 256 * 384;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "consumer tile must be whole 32x32 blocks");
  static_assert(A_INS * NCOPY * 1024 == A_BYTES && B_INS * NCOPY * 1024 == B_BYTES, "whole copies");
  static_assert(NSTAGE >= 3, "need at least three stages");
  static_assert((PREF - 1) * NVM <= 63, "vmcnt range");
};

// LDS stage of K step kt (kt >= 0): unsigned modulo where the ring is a power of
// two (one scalar AND), signed otherwise (the compiler's multiply-shift for the
// unsigned form of a 5-stage ring lands in vector registers).
template <class C>
__device__ __forceinline__ int stage_of(int kt) {
  return (C::NSTAGE & (C::NSTAGE - 1)) == 0 ? (int)((unsigned)kt % C::NSTAGE) : kt % C::NSTAGE;
}

// One copying wave's share of every K step's copies.  Every in-range offset of
// one K step stays below the record-count cap of make_rsrc: the largest is row
// 383 of a 384-row panel whose rows are 2^21 elements (the feature-dimension
// limit) apart, 383 * 2^22 + 1008 bytes < 2^31 - 16.
template <class C, bool AK, bool BKC>
struct Copier {
  const char* a_base;
  const char* b_base;
  int64_t a_total, b_total, a_step, b_step;
  // Record counts in 32-bit arithmetic: bytes from step kt's base to the end of
  // the operand are total - kt * step; the first *_hi steps have more than OOB
  // (clamped to OOB: every in-range offset is then inside the operand), after
  // that the count fits in an int and is taken from the low 32 bits.
  int a_hi, b_hi, a_tot32, b_tot32, a_step32, b_step32;
  int a_off[C::A_INS], a_kc[C::A_INS], b_off[C::B_INS], b_kc[C::B_INS];
  unsigned smem_addr;
  int cw, K;
  // The step whose copies issue() makes (kcur), its two buffer resources and
  // unclamped 32-bit remaining byte counts, advanced one step at a time.
  int kcur, a_rem, b_rem;
  unsigned st_cur;   // LDS address of stage kcur % NSTAGE
  i32x4 ra, rb;

  __device__ __forceinline__ void init(const GemmArgs& g, int m0, int n0, int cw_, int lane, const char* smem) {
    constexpr int KCH = KT / 8;  // 16-byte chunks per row of a K-contiguous panel
    cw = cw_;
    K = g.K;
    a_base = (const char*)g.A + 2 * (AK ? (int64_t)m0 * g.lda : (int64_t)m0);
    b_base = (const char*)g.B + 2 * (BKC ? (int64_t)n0 * g.ldb : (int64_t)n0);
    a_total = 2 * ((AK ? (int64_t)g.M : (int64_t)g.K) * g.lda - (AK ? (int64_t)m0 * g.lda : m0));
    b_total = 2 * ((BKC ? (int64_t)g.N : (int64_t)g.K) * g.ldb - (BKC ? (int64_t)n0 * g.ldb : n0));
    a_step = AK ? 2 * KT : 2 * (int64_t)KT * g.lda;
    b_step = BKC ? 2 * KT : 2 * (int64_t)KT * g.ldb;
    a_hi = a_total > OOB ? (int)((a_total - OOB - 1) / a_step + 1) : 0;
    b_hi = b_total > OOB ? (int)((b_total - OOB - 1) / b_step + 1) : 0;
    a_tot32 = (int)(uint32_t)a_total;
    b_tot32 = (int)(uint32_t)b_total;
    a_step32 = (int)a_step;
    b_step32 = (int)b_step;
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) {
      const int q = (cw * C::A_INS + j) * 64 + lane;  // 16-byte chunk index in the stage's A panel
      if (AK) {
        const int r = q / KCH, sl = q % KCH, c = sl ^ ((r >> 2) & 3);
        a_off[j] = r * (int)g.lda * 2 + c * 16;
        a_kc[j] = c * 8;
      } else {
        constexpr int CPR = C::BM / 8;
        const int r = q / CPR, sl = q % CPR, c = sl ^ mn_swz<C::BM>(r);
        a_off[j] = (m0 + c * 8 < g.M) ? r * (int)g.lda * 2 + c * 16 : OOB;
        a_kc[j] = 0;
      }
    }
#pragma unroll
    for (int j = 0; j < C::B_INS; ++j) {
      const int q = (cw * C::B_INS + j) * 64 + lane;
      if (BKC) {
        const int r = q / KCH, sl = q % KCH, c = sl ^ ((r >> 2) & 3);
        b_off[j] = r * (int)g.ldb * 2 + c * 16;
        b_kc[j] = c * 8;
      } else {
        constexpr int CPR = C::BN / 8;
        const int r = q / CPR, sl = q % CPR, c = sl ^ mn_swz<C::BN>(r);
        b_off[j] = (n0 + c * 8 < g.N) ? r * (int)g.ldb * 2 + c * 16 : OOB;
        b_kc[j] = 0;
      }
    }
    smem_addr = lds_address(smem);
  }

  // Make step kt the one issue() copies.
  __device__ __forceinline__ void start(int kt) {
    kcur = kt;
    st_cur = smem_addr + stage_of<C>(kt) * C::STAGE;
    a_rem = (int)((uint32_t)a_tot32 - (uint32_t)kt * (uint32_t)a_step32);
    b_rem = (int)((uint32_t)b_tot32 - (uint32_t)kt * (uint32_t)b_step32);
    ra = make_rsrc_n(a_base + kt * a_step, kt < a_hi ? OOB : max(0, a_rem));
    rb = make_rsrc_n(b_base + kt * b_step, kt < b_hi ? OOB : max(0, b_rem));
  }
  // On to step kcur + 1: the bases move by one step (a 64-bit add in the first
  // two resource words; a buffer's base stays below 2^48), the counts shrink.
  __device__ __forceinline__ void advance() {
    ++kcur;
    st_cur = st_cur + C::STAGE == smem_addr + C::NSTAGE * C::STAGE ? smem_addr : st_cur + C::STAGE;
    const uint64_t a = ((uint64_t)(uint32_t)ra[1] << 32 | (uint32_t)ra[0]) + (uint64_t)a_step;
    const uint64_t b = ((uint64_t)(uint32_t)rb[1] << 32 | (uint32_t)rb[0]) + (uint64_t)b_step;
    a_rem -= a_step32;
    b_rem -= b_step32;
    ra[0] = (int)(uint32_t)a;
    ra[1] = (int)(uint32_t)(a >> 32);
    ra[2] = kcur < a_hi ? OOB : max(0, a_rem);
    rb[0] = (int)(uint32_t)b;
    rb[1] = (int)(uint32_t)(b >> 32);
    rb[2] = kcur < b_hi ? OOB : max(0, b_rem);
  }

  // Copy u (0 <= u < NVM) of K step kcur into LDS stage kcur % NSTAGE.  Past the
  // last step the copies read only zeros into a stage that is not used again.
  // TAIL: the step may reach past K (K-contiguous chunks at or past K read as
  // zeros); without it the caller guarantees (kcur + 1) * KT <= K.
  template <bool TAIL = true>
  __device__ __forceinline__ void issue(int u) const {
    const int k0 = kcur * KT;
    const unsigned st = st_cur;
    if (u < C::A_INS) {
      const int j = u;
      lds_dma16(ra, (TAIL && AK && k0 + a_kc[j] >= K) ? OOB : a_off[j], st + (cw * C::A_INS + j) * 1024);
    } else {
      const int j = u - C::A_INS;
      lds_dma16(rb, (TAIL && BKC && k0 + b_kc[j] >= K) ? OOB : b_off[j], st + C::A_BYTES + (cw * C::B_INS + j) * 1024);
    }
  }
};

// A consumer wave's MFMA operand reads from an LDS stage.
template <class C, bool AK, bool BKC, typename E>
struct Reader {
  using V8 = typename Vec<E>::v8;
  using V4 = typename Vec<E>::v4;
  int wm, wn, l32, hi, kswz, tr_row, tr_col, tr_swz_a, tr_swz_b;
  // K-contiguous operands: this lane's byte offset in the stage for k slice s
  // of its first fragment; fragment i sits 32 i rows (an immediate) further.
  int ka[KT / 16], kb[KT / 16];
  // M/N-contiguous operands: this lane's byte offset in the stage of the first
  // transposing read of fragment i (j) in k slice 0; slice s and the second read
  // are immediates further (16 s and 16 s + 4 k-rows).
  int ma[C::FM], mb[C::FN];

  __device__ __forceinline__ void init(int wave, int lane) {
    wm = wave / C::CN;
    wn = wave % C::CN;
    l32 = lane & 31;
    hi = lane >> 5;
    kswz = (l32 >> 2) & 3;                      // K-contig slot swizzle of this lane's row
#pragma unroll
    for (int s = 0; s < KT / 16; ++s) {
      const int slot = (2 * s + hi) ^ kswz;     // rows 32 i apart have the same swizzle
      ka[s] = (wm * C::WM + l32) * (KT * 2) + slot * 16;
      kb[s] = C::A_BYTES + (wn * C::WN + l32) * (KT * 2) + slot * 16;
    }
    const int grp = lane >> 4, i16 = lane & 15; // transpose read: 16-lane group, lane in it
    tr_row = 8 * (grp >> 1) + (i16 >> 2);
    tr_col = 16 * (grp & 1) + 4 * (i16 & 3);
    tr_swz_a = mn_swz<C::BM>(i16 >> 2);
    tr_swz_b = mn_swz<C::BN>(i16 >> 2);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int col = wm * C::WM + 32 * i + tr_col;
      ma[i] = tr_row * (C::BM * 2) + ((col >> 3) ^ tr_swz_a) * 16 + (col & 7) * 2;
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = wn * C::WN + 32 * j + tr_col;
      mb[j] = C::A_BYTES + tr_row * (C::BN * 2) + ((col >> 3) ^ tr_swz_b) * 16 + (col & 7) * 2;
    }
  }
  __device__ __forceinline__ V8 frag_k(const char* panel, int row0, int s) const {
    const int r = row0 + l32;
    const int slot = (2 * s + hi) ^ kswz;
    return *(const V8*)(panel + r * (KT * 2) + slot * 16);
  }
  __device__ __forceinline__ V8 frag_mn(const char* panel, int row_bytes, int swz, int col0, int s) const {
    const int col = col0 + tr_col;
    const int slot = (col >> 3) ^ swz;
    const char* p0 = panel + (16 * s + tr_row) * row_bytes + slot * 16 + (col & 7) * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    const i16x4 hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p0 + 4 * row_bytes));
    const V4 lo_b = __builtin_bit_cast(V4, lo);
    const V4 hi_b = __builtin_bit_cast(V4, hv);
    V8 v;
    v[0] = lo_b[0]; v[1] = lo_b[1]; v[2] = lo_b[2]; v[3] = lo_b[3];
    v[4] = hi_b[0]; v[5] = hi_b[1]; v[6] = hi_b[2]; v[7] = hi_b[3];
    return v;
  }
  // The transposing reads of one M/N-contiguous fragment from its lane offset.
  __device__ __forceinline__ V8 frag_mn_at(const char* p0, int row_bytes) const {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    const i16x4 hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p0 + 4 * row_bytes));
    const V4 lo_b = __builtin_bit_cast(V4, lo);
    const V4 hi_b = __builtin_bit_cast(V4, hv);
    V8 v;
    v[0] = lo_b[0]; v[1] = lo_b[1]; v[2] = lo_b[2]; v[3] = lo_b[3];
    v[4] = hi_b[0]; v[5] = hi_b[1]; v[6] = hi_b[2]; v[7] = hi_b[3];
    return v;
  }
  // Operands of 16-wide k slice s of K step kt.
  __device__ __forceinline__ void load(const char* smem, int kt, int s, V8* fa, V8* fb) const {
    load_at(smem + stage_of<C>(kt) * C::STAGE, s, fa, fb);
  }
  // The same from the stage at sa.
  __device__ __forceinline__ void load_at(const char* sa, int s, V8* fa, V8* fb) const {
    const char* sb = sa + C::A_BYTES;
    // (the producer/consumer kernels keep the per-fragment form: in their
    // register budget the per-slice bases measured slower)
    constexpr bool BASES = C::NPROD == 0;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      fa[i] = !AK ? (BASES ? frag_mn_at(sa + ma[i] + 16 * s * (C::BM * 2), C::BM * 2)
                           : frag_mn(sa, C::BM * 2, tr_swz_a, wm * C::WM + 32 * i, s))
                  : BASES ? *(const V8*)(sa + ka[s] + 32 * i * (KT * 2)) : frag_k(sa, wm * C::WM + 32 * i, s);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      fb[j] = !BKC ? (BASES ? frag_mn_at(sa + mb[j] + 16 * s * (C::BN * 2), C::BN * 2)
                            : frag_mn(sb, C::BN * 2, tr_swz_b, wn * C::WN + 32 * j, s))
                   : BASES ? *(const V8*)(sa + kb[s] + 32 * j * (KT * 2)) : frag_k(sb, wn * C::WN + 32 * j, s);
  }
};

// Column sums of B over K, computed alongside a weight gradient whose B
// operand (stored [K x N]) is the output gradient dY: the sums are the bias
// gradient db = sum_t dY, so dY is not read a second time.  The tiles_m tiles
// of a column panel split K between them: tile row tm adds the K steps tm,
// tm + tiles_m, ... of its B panel, while that step is in LDS anyway.  Lane L
// of the first BN consumer lanes owns columns 4 (L / 4) .. + 3 of the panel
// and k-rows j, j + 4, ..., j + 28 (j = L % 4) of a step; its 4 fp32 sums stay
// in registers over the K loop (4, not 8: the big tiles have no registers to
// spare).  At the end the 4 lanes of a column quad are added in a fixed order
// and the tile writes its partial row (row tm); a second pass adds the
// tiles_m rows in order.
template <class C, typename E>
struct BColSum {
  using V4 = typename Vec<E>::v4;
  static constexpr int LANES = C::BN;     // one lane per 4 columns and 8 k-rows
  static_assert(LANES % 64 == 0 && LANES <= 64 * C::NCONS, "column-sum lanes are whole consumer waves");
  static_assert(KT == 32, "eight k-rows per lane");
  float s[4];
  int next;   // next K step this tile adds (wave-uniform)
  bool on;    // wave-uniform: sums wanted and this wave takes part

  // kbeg: the first K step of this workgroup's range (0, or the second half's).
  __device__ __forceinline__ void init(const GemmArgs& g, int wave, int tm, int tiles_m, int kbeg) {
    on = g.colsum != nullptr && wave * 64 < LANES;
    next = kbeg > tm ? tm + (kbeg - tm + tiles_m - 1) / tiles_m * tiles_m : tm;
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = 0.0f;
  }
  // Add K step kt (in LDS) when it is this tile's.
  __device__ __forceinline__ void step(const char* smem, int kt, int tiles_m, int wave, int lane) {
    if (!on || kt != next) return;
    next += tiles_m;
    // The address is derived here, inside the branch, rather than hoisted above
    // the K loop where it would hold registers that the main loop needs.
    asm volatile("" : "+v"(lane));
    const int L = wave * 64 + lane, q = L >> 2, j = L & 3;
    // rows j + 4 u all have row j's chunk swizzle (it depends on the row mod 4)
    const int off = j * (C::BN * 2) + (((q >> 1) ^ mn_swz<C::BN>(j)) * 16) + (q & 1) * 8;
    const char* sb = smem + stage_of<C>(kt) * C::STAGE + C::A_BYTES + off;
    V4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const V4*)(sb + u * 4 * C::BN * 2);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += (float)v[u][e];
  }
  // Add the 4 lanes of each column quad and write the tile's partial row (row
  // tm, or tiles_m + tm for the second K half of a split launch).
  __device__ __forceinline__ void finish(const GemmArgs& g, int tm, int n0, int wave, int lane) {
    if (!on) return;
#pragma unroll
    for (int m = 1; m < 4; m <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += __shfl_xor(s[e], m);
    const int n = n0 + 4 * ((wave * 64 + lane) >> 2);
    if ((lane & 3) == 0 && n < g.N) *(f32x4*)(g.colsum + (int64_t)tm * g.N + n) = f32x4{s[0], s[1], s[2], s[3]};
  }
};

// Epilogue of one consumer wave, through LDS.  The accumulators hold, per lane,
// 4 runs of 4 consecutive columns of one row (block (i, j), lane: row l32,
// columns 32 j + 8 q + 4 (lane / 32) + 0..3); stored directly, every store
// instruction would write 16-byte pieces of 32 different rows.  Instead each
// wave stages 32-row strips of its sub-tile in the (now idle) LDS ring --
// rows padded so the register-order accesses fall in different banks -- and
// moves them between LDS and memory as 16-byte chunks with consecutive lanes
// along a row.  The GeLU' operand Z comes in the same way.
template <class C, int EPI, typename E>
__device__ __forceinline__ void epilogue(const GemmArgs& g, f32x16 (&acc)[C::FM][C::FN], int m0, int n0,
                                         int wave, int lane, char* smem) {
  using V4 = typename Vec<E>::v4;
  using V8 = typename Vec<E>::v8;
  // The coordinates are passed through empty asm so that the compiler derives the
  // epilogue addresses here instead of hoisting them above the K loop, where they
  // would hold registers for its whole duration.
  asm volatile("" : "+v"(lane));
  asm volatile("" : "+s"(m0), "+s"(n0), "+s"(wave));
  constexpr bool F32 = EPI == EPI_F32;
  constexpr int ES = F32 ? 4 : 2;                    // output element bytes
  constexpr int ROWB = C::WN * ES;                   // bytes of a strip row
  constexpr int PITCH = ROWB + (F32 ? 16 : 8);       // padded LDS row pitch
  constexpr int CPR = ROWB / 16;                     // 16-byte chunks per row
  constexpr int NCH = 32 * CPR;                      // chunks per strip
  constexpr int NIT = (NCH + 63) / 64;
  static_assert(ROWB % 16 == 0, "strip rows are whole 16-byte chunks");
  static_assert(C::NCONS * 32 * PITCH * (EPI == EPI_DGELU_H ? 2 : 1) <= C::NSTAGE * C::STAGE, "strips fit in the ring");
  char* strip = smem + wave * 32 * PITCH;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = wave / C::CN, wn = wave % C::CN;
  const int col0 = n0 + wn * C::WN;

  // Strip rows <-> memory, 16-byte chunks (cols past N and rows past M skipped).
  auto to_mem_from = [&](const char* sbase, void* base, int64_t ld, int row0) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = it * 64 + lane;
      if (NCH % 64 != 0 && c >= NCH) continue;
      const int r = c / CPR, cc = c % CPR;
      const int m = row0 + r, n = col0 + cc * (16 / ES);
      if (m >= g.M || n >= g.N) continue;
      const char* p = sbase + r * PITCH + cc * 16;
      if (F32) {
        f32x4 v = *(const f32x4*)p;
        float* dst = (float*)base + (int64_t)m * ld + n;
        if (g.accumulate) {
          const f32x4 old = *(const f32x4*)dst;
          v[0] += old[0]; v[1] += old[1]; v[2] += old[2]; v[3] += old[3];
        }
        // Non-temporal: the fp32 parameter gradients are not read again by
        // the kernels that follow, and streaming them past the caches keeps
        // those kernels' operands resident (+0.45% on the layer step).
        __builtin_nontemporal_store(v, (f32x4*)dst);
      } else {
        *(V8*)((E*)base + (int64_t)m * ld + n) = *(const V8*)p;
      }
    }
  };
  auto to_mem = [&](void* base, int64_t ld, int row0) { to_mem_from(strip, base, ld, row0); };
  auto from_mem = [&](const void* base, int64_t ld, int row0) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = it * 64 + lane;
      if (NCH % 64 != 0 && c >= NCH) continue;
      const int r = c / CPR, cc = c % CPR;
      const int m = row0 + r, n = col0 + cc * 8;
      V8 v{};
      if (m < g.M && n < g.N) v = *(const V8*)((const E*)base + (int64_t)m * ld + n);
      *(V8*)(strip + r * PITCH + cc * 16) = v;
    }
  };
  // This lane's 4 values of run (j, q) in the strip.
  auto at = [&](int j, int q) { return strip + l32 * PITCH + (32 * j + 8 * q + 4 * hh) * ES; };

#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int row0 = m0 + wm * C::WM + 32 * i;
    if (F32) {
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f32x4*)at(j, q) = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      to_mem(g.C, g.ldc, row0);
      continue;
    }
    if (EPI == EPI_DGELU || EPI == EPI_DGELU_H) {
      from_mem(g.aux, g.ldaux, row0);
      if (EPI == EPI_DGELU_H) {
        // dZ = acc * GeLU'(Z) over Z in the strip and H = GeLU(Z) into a second
        // strip (above the first set in the idle ring), from one evaluation of
        // erf and the Gaussian per element.
        char* strip2 = smem + (C::NCONS + wave) * 32 * PITCH;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const V4 zz = *(const V4*)at(j, q);
            V4 hv, dz;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float z = (float)zz[e];
              const GeluParts gp = gelu_parts(z);
              dz[e] = (E)(acc[i][j][4 * q + e] * __builtin_fmaf(z, gp.pdf, gp.cdf));
              hv[e] = (E)(z * gp.cdf);
            }
            *(V4*)at(j, q) = dz;
            *(V4*)(strip2 + (at(j, q) - strip)) = hv;
          }
        to_mem_from(strip2, g.C2, g.ldc2, row0);
        to_mem(g.C, g.ldc, row0);
        continue;
      }
    }
    // z = acc (+ bias) for run (j, q)
    auto zval = [&](int j, int q, float* z) {
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = acc[i][j][4 * q + e];
      const int n = col0 + 32 * j + 8 * q + 4 * hh;
      if ((EPI == EPI_STORE || EPI == EPI_BIAS_GELU) && g.bias != nullptr && n < g.N) {
        const V4 b = *(const V4*)((const E*)g.bias + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] += (float)b[e];
      }
    };
    if (EPI == EPI_BIAS_GELU && g.C2 != nullptr) {
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float z[4];
          zval(j, q, z);
          V4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (E)z[e];
          *(V4*)at(j, q) = o;
        }
      to_mem(g.C2, g.ldc2, row0);
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float z[4];
        zval(j, q, z);
        if (EPI == EPI_DGELU) {
          const V4 zz = *(const V4*)at(j, q);   // the saved pre-activation, staged above
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] *= gelu_grad_f((float)zz[e]);
        }
        V4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (E)(EPI == EPI_BIAS_GELU ? gelu_f(z[e]) : z[e]);
        *(V4*)at(j, q) = o;
      }
    to_mem(g.C, g.ldc, row0);
  }
}

// One workgroup's tile: workgroup id bid0 of the product g, LDS ring smem.
template <class C, bool AK, bool BKC, int EPI, typename E>
__device__ __forceinline__ void gemm_tile(GemmArgs g, int bid0, char* smem) {
  using V8 = typename Vec<E>::v8;
  constexpr int FM = C::FM, FN = C::FN, NVM = C::NVM, PREF = C::PREF;
  constexpr int NS = KT / 16;             // 16-wide k slices per step
  constexpr int LB = (NS - 1) & 1;        // operand buffer of the last slice (double buffering)
  // Rows of the last slice's MFMAs issued before the step's barrier; the rest
  // run after it, while step kt+1's first operands are read.  Half, except in
  // the shared kernels on the weight-gradient layout (both operands read with
  // transposing reads), where one row before and the rest after measured 1.5%
  // faster (and the other layouts 1% slower).
  constexpr int FM_HALF = (C::NPROD == 0 && !AK && !BKC) ? 1 : (FM / 2 > 0 ? FM / 2 : 1);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int tiles_m = (g.M + C::BM - 1) / C::BM;
  const int tiles_n = (g.N + C::BN - 1) / C::BN;
  // K split (weight gradients whose tiles fill at most half of the CUs, with
  // g.kpart set by the launcher): workgroups [tiles, 2 tiles) take the second
  // half of the K steps and write their partial to g.kpart.
  int bid = bid0, part = 0;
  if (EPI == EPI_F32 && g.kpart != nullptr && bid >= tiles_m * tiles_n) {
    bid -= tiles_m * tiles_n;
    part = 1;
  }
  int tm, tn;
  tile_coords(bid, tiles_m, tiles_n, g.group_m, tm, tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;
  const int nk_all = (g.K + KT - 1) / KT;
  const bool ksplit = EPI == EPI_F32 && g.kpart != nullptr;
  const int kbeg = ksplit && part ? nk_all / 2 : 0;             // this workgroup's K steps [kbeg, nk)
  const int nk = ksplit && !part ? nk_all / 2 : nk_all;

  if constexpr (C::NPROD > 0) {
    if (wave >= C::NCONS) {
      // -------------------------------------------------------- producer wave
      Copier<C, AK, BKC> cp;
      cp.init(g, m0, n0, wave - C::NCONS, lane, smem);
      cp.start(kbeg);
#pragma unroll
      for (int p = 0; p < PREF; ++p) {
#pragma unroll
        for (int u = 0; u < NVM; ++u) cp.issue(u);
        cp.advance();
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((PREF - 1) * NVM));  // step kbeg landed
      __syncthreads();
      // steps before ksafe prefetch a step that lies wholly inside K: no tail check
      const int ksafe = (AK && BKC) ? max(kbeg, min(nk, g.K / KT - PREF)) : kbeg;
      auto pstep = [&](int kt, auto tail) {
#pragma unroll
        for (int u = 0; u < NVM; ++u) cp.template issue<decltype(tail)::value>(u);   // step kt + PREF
        cp.advance();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((PREF - 1) * NVM));  // step kt+1 landed
        __syncthreads();
      };
      int kt = kbeg;
      if constexpr (AK && BKC)
        for (; kt < ksafe; ++kt) pstep(kt, std::false_type{});
      for (; kt < nk; ++kt) pstep(kt, std::true_type{});
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no copy into this workgroup's LDS outlives it
      return;
    }
  }

  // ------------------------------------------------------------ consumer wave
  Reader<C, AK, BKC, E> rd;
  rd.init(wave, lane);
  constexpr bool CS = C::CSUM && !BKC && EPI == EPI_F32;   // B stored [K x N]: its column sums can ride along
  BColSum<C, E> cs;
  if constexpr (CS) cs.init(g, wave, tm, tiles_m, kbeg);
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto mfma = [&](const V8* fa_, const V8* fb_, int i, int j) { acc[i][j] = mfma32(fb_[j], fa_[i], acc[i][j]); };

  if constexpr (C::NPROD > 0) {
    __syncthreads();  // step kbeg is in LDS
    V8 fa[2][FM], fb[2][FN];
    // stages of steps kt and kt + 1, advanced around the ring once per step
    const char* const ring_end = smem + C::NSTAGE * C::STAGE;
    const char* st_k = smem + stage_of<C>(kbeg) * C::STAGE;
    const char* st_n = st_k + C::STAGE == ring_end ? smem : st_k + C::STAGE;
    rd.load_at(st_k, 0, fa[0], fb[0]);
    for (int kt = kbeg; kt < nk; ++kt) {
      if constexpr (AK && BKC) __builtin_amdgcn_s_setprio(1);  // see the shared kernel below
#pragma unroll
      for (int s = 0; s < NS - 1; ++s) {
        rd.load_at(st_k, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mfma(fa[s & 1], fb[s & 1], i, j);
      }
      // Last slice: part of its MFMAs, the barrier that publishes step kt+1 (and
      // releases step kt's stage to the producers), then step kt+1's first
      // operands are read while the rest run.
#pragma unroll
      for (int i = 0; i < FM_HALF; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma(fa[LB], fb[LB], i, j);
      if constexpr (AK && BKC) __builtin_amdgcn_s_setprio(0);
      if constexpr (CS) cs.step(smem, kt, tiles_m, wave, lane);
      __syncthreads();
      rd.load_at(st_n, 0, fa[LB ^ 1], fb[LB ^ 1]);
      st_k = st_n;
      st_n = st_n + C::STAGE == ring_end ? smem : st_n + C::STAGE;
#pragma unroll
      for (int i = FM_HALF; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma(fa[LB], fb[LB], i, j);
    }
  } else {
    // The copying waves (all 8, or the first NCOPY) also issue their share of
    // the copies, spread over the MFMAs that precede each step's barrier (the
    // other wave on the SIMD keeps the matrix pipe busy while a copy holds this
    // one up).  A wave that issues none waits on an empty vmcnt.
    //
    // Wave priority: a wave raises its issue priority while it works through a
    // step's MFMAs and drops it for the wait, the barrier and the next step's
    // first operand reads.  The barrier leaves the two waves of a SIMD in step;
    // the priority lets one of them run ahead, so that its MFMAs fill the
    // matrix pipe while the other waits on LDS (measured: +3-4% on the
    // both-K-contiguous layout, +0.5% on TN, none on NN).  The split kernels do
    // the same for their consumers on the both-K-contiguous layout only (+2%
    // there; it cost 1.5% on NN).
    constexpr bool ALL_COPY = C::NCOPY == C::NCONS;
    const bool copier = ALL_COPY || wave < C::NCOPY;
    Copier<C, AK, BKC> cp;
    cp.init(g, m0, n0, wave, lane, smem);
    cp.start(kbeg);
#pragma unroll
    for (int p = 0; p < PREF; ++p) {
      if (copier) {
#pragma unroll
        for (int u = 0; u < NVM; ++u) cp.issue(u);
      }
      cp.advance();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((PREF - 1) * NVM));  // step kbeg landed
    __syncthreads();
    V8 fa[FM], fb[FN];
    // cpy: this wave issues copies (a constant: waves that copy and waves that
    // do not run separate copies of the loop, so no copy sits behind a branch);
    // fmh: rows of the last slice's MFMAs before the barrier
    auto kstep = [&](int kt, auto tail, auto cpy, auto fmh) {
      constexpr bool TAIL = decltype(tail)::value;
      constexpr bool CPY = decltype(cpy)::value;
      constexpr int FMH = decltype(fmh)::value;
      constexpr int PRE_MF = FM * FN * (NS - 1) + FMH * FN;   // MFMAs before the barrier
      static_assert(!CPY || PRE_MF >= NVM, "not enough MFMAs to spread the copies over");
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        rd.load(smem, kt, s, fa, fb);
        const int i_end = (s == NS - 1) ? FMH : FM;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < i_end; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            mfma(fa, fb, i, j);
            const int t = s * FM * FN + i * FN + j;
#pragma unroll
            for (int u = 0; u < NVM; ++u)
              if ((u * PRE_MF) / NVM == t) {
                if constexpr (CPY) cp.template issue<TAIL>(u);   // step kt + PREF
              }
          }
      }
      __builtin_amdgcn_s_setprio(0);
      if constexpr (CPY) cp.advance();
      if constexpr (CS) cs.step(smem, kt, tiles_m, wave, lane);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((PREF - 1) * NVM));  // step kt+1 landed
      __syncthreads();
#pragma unroll
      for (int i = FMH; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma(fa, fb, i, j);
    };
    // Steps before ksafe prefetch a step that lies wholly inside K: no tail check
    // (both operands K-contiguous, where every copy would carry it; on the other
    // layouts the second copy of the loop costs registers).
    const int ksafe = (AK && BKC) ? max(kbeg, min(nk, g.K / KT - PREF)) : kbeg;
    auto kloop = [&](auto cpy, auto fmh) {
      int kt = kbeg;
      if constexpr (AK && BKC)
        for (; kt < ksafe; ++kt) kstep(kt, std::false_type{}, cpy, fmh);
      for (; kt < nk; ++kt) kstep(kt, std::true_type{}, cpy, fmh);
    };
    // The first wave on each SIMD (waves 0-3, dispatched first) wins the matrix
    // pipe while both have MFMAs ready, reaches the barrier ~460 cycles before
    // the second (a cycle-stamped build of the 256 x 384 data gradient) and
    // waits there.  Where A is K-contiguous and four rows of fragments are held,
    // the second wave runs one row fewer before the barrier (and one more after
    // it): 2 / 1 rows measured 0.7-1.7% faster than 2 / 2 on the NN / NT
    // kernels (3 / 1 no better, 4 / 0 slower); the weight-gradient kernels keep
    // one row on both waves (moving rows there was mixed).
    constexpr int FHA = FM_HALF;
    constexpr int FHB = (AK && FM >= 4) ? FM_HALF - 1 : FM_HALF;
    static_assert(C::NCOPY == C::NCONS || C::NCOPY == 4, "copying waves are all, or the first on each SIMD");
    if (wave < 4) kloop(std::true_type{}, std::integral_constant<int, FHA>{});
    else if constexpr (ALL_COPY) kloop(std::true_type{}, std::integral_constant<int, FHB>{});
    else kloop(std::false_type{}, std::integral_constant<int, FHB>{});
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no copy into this workgroup's LDS outlives it
  }

  if constexpr (CS) cs.finish(g, tm + part * tiles_m, n0, wave, lane);
  __syncthreads();  // every consumer is done with the ring (producer copies have drained)
  if (EPI == EPI_F32 && part) {
    // the second K half: its partial to g.kpart (ld = N), added to C afterwards
    g.C = g.kpart;
    g.ldc = g.N;
    g.accumulate = 0;
  }
  epilogue<C, EPI, E>(g, acc, m0, n0, wave, lane, smem);
}

template <class C, bool AK, bool BKC, int EPI, typename E>
__global__ void __attribute__((amdgpu_flat_work_group_size(C::NT, C::NT),
                               amdgpu_waves_per_eu(C::WAVES_PER_EU, C::WAVES_PER_EU)))
gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGE];
  gemm_tile<C, AK, BKC, EPI, E>(g, (int)blockIdx.x, smem);
}

// Two independent products in one launch: workgroups [0, n1) take the tiles
// of g1, the rest those of g2.  The dispatcher hands out workgroups in id
// order, so g1's (long) tiles start first, each on a CU of its own, and g2's
// fill the other CUs and then those that g1 releases.
template <class C1, bool AK1, bool BKC1, int EPI1, class C2, bool AK2, bool BKC2, int EPI2, typename E>
__global__ void __attribute__((amdgpu_flat_work_group_size(C1::NT, C1::NT),
                               amdgpu_waves_per_eu(C1::WAVES_PER_EU, C1::WAVES_PER_EU)))
gemm_pair_kernel(GemmArgs g1, GemmArgs g2, int n1) {
  static_assert(C1::NT == C2::NT && C1::WAVES_PER_EU == C2::WAVES_PER_EU, "one workgroup shape");
  constexpr int L1 = C1::NSTAGE * C1::STAGE, L2 = C2::NSTAGE * C2::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[L1 > L2 ? L1 : L2];
  if ((int)blockIdx.x < n1) gemm_tile<C1, AK1, BKC1, EPI1, E>(g1, (int)blockIdx.x, smem);
  else gemm_tile<C2, AK2, BKC2, EPI2, E>(g2, (int)blockIdx.x - n1, smem);
}

// Tile menu: split kernels (8 consumer + 4 producer waves) and shared kernels
// (8 waves that copy and compute).
using T256x192 = Cfg<256, 192, 4, 4>;
using T192x256 = Cfg<192, 256, 4, 2>;
using T256x128 = Cfg<256, 128, 4, 4>;
using T128x256 = Cfg<128, 256, 4, 2>;
using T128x128 = Cfg<128, 128, 4, 2>;
using T256x384 = Cfg<256, 384, 0, 2>;
using T384x256 = Cfg<384, 256, 0, 4>;
using T192x384 = Cfg<192, 384, 0, 2, 4>;  // 36 KiB per K step: 4 copying waves (one per SIMD) x 9 copies
using T256x256 = Cfg<256, 256, 0, 2>;     // 128 x 64 per wave, five 32 KiB stages

template <class C, bool AK, bool BKC, int EPI, typename E>
const char* kname() {
  static const std::string s = std::string("gemm_") + Vec<E>::name + "_" + (AK ? "n" : "t") + (BKC ? "t" : "n") + "_" +
                               (EPI == EPI_STORE ? "store" : EPI == EPI_BIAS_GELU ? "bias_gelu"
                                : EPI == EPI_DGELU ? "dgelu" : EPI == EPI_DGELU_H ? "dgelu_h" : "f32") +
                               "_" + std::to_string(C::BM) + "x" + std::to_string(C::BN);
  return s.c_str();
}

// Rows of tiles per group in the tile order.  The 32 workgroups an XCD runs at
// once cover about g tile rows x 32/g tile columns; their L2 fetches g row
// panels of A (BM x K each) and 32/g column panels of B (K x BN each), so g is
// chosen to minimise g * BM + (32 / g) * BN.
int choose_group_m(int tiles_m, int bm, int bn) {
  int best = 1;
  double best_cost = 1e300;
  for (int gm = 1; gm <= 32; gm *= 2) {
    if (gm > tiles_m) break;
    const double cost = (double)gm * bm + 32.0 / gm * bn;
    if (cost < best_cost * 0.999) { best_cost = cost; best = gm; }
  }
  return best;
}

template <class C, bool AK, bool BKC>
int group_for(int tiles_m) {
  int gm = choose_group_m(tiles_m, C::BM, C::BN);
  // Measured exceptions to the estimate: the 192 x 384 weight-gradient tile
  // (both operands M/N-contiguous) runs 2% faster with twice the height
  // (longer contiguous runs of each token row per K step), the 256 x 384
  // data-gradient tile (both K-contiguous) 0.6-0.9% faster with half; the
  // other kernels ran 1-3% slower with either.
  if (!AK && !BKC && C::BM == 192 && 2 * gm <= tiles_m) gm *= 2;
  if (AK && BKC && C::BM == 256 && C::BN == 384 && gm > 1) gm /= 2;
  return gm;
}

template <class C, bool AK, bool BKC, int EPI, typename E>
hipError_t launch_tile(const GemmArgs& g_in, hipStream_t s, const char** name) {
  *name = kname<C, AK, BKC, EPI, E>();
  GemmArgs g = g_in;
  const int tiles_m = (g.M + C::BM - 1) / C::BM, tiles_n = (g.N + C::BN - 1) / C::BN;
  g.group_m = group_for<C, AK, BKC>(tiles_m);
  const int parts = (EPI == EPI_F32 && g.kpart != nullptr) ? 2 : 1;   // K split: two workgroups per tile
  hipLaunchKernelGGL((gemm_kernel<C, AK, BKC, EPI, E>), dim3(tiles_m * tiles_n * parts), dim3(C::NT), 0, s, g);
  return hipGetLastError();
}

// The second pass of a K-split weight gradient: C[M x N] (row stride ldc) +=
// P[M x N] (row stride N), 4 fp32 per work-item.  C then holds (C's first-half
// value) + (second half), one fixed order.
__global__ void __launch_bounds__(256) kpart_add_kernel(float* C, int64_t ldc, const float* P, int M, int N) {
  const int64_t nq = N / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * nq) return;
  const int64_t r = i / nq, c = (i - r * nq) * 4;
  f32x4 v = *(const f32x4*)(C + r * ldc + c);
  const f32x4 q = *(const f32x4*)(P + r * N + c);
  v[0] += q[0];
  v[1] += q[1];
  v[2] += q[2];
  v[3] += q[3];
  *(f32x4*)(C + r * ldc + c) = v;
}

// Tile shape: the one with the least estimated time, counting whole waves of
// tiles over the 256 CUs (one workgroup per CU) and a per-tile efficiency that
// grows with the tile (fewer bytes moved per FLOP).  256 x 256 moves as many
// bytes per FLOP between L2 and LDS as 192 x 384 and fills whole waves where
// that one leaves a partial wave (the 1.3B MLP's 4096 x 8192 products with
// K = 2048 and its weight gradients: +7% and +3% in a same-box A/B).
struct TileChoice { int bm, bn; };

TileChoice choose_tile(int M, int N, bool shared_tiles = true) {
  static const struct { int bm, bn; double eff; } cand[] = {
      {256, 384, 1.12}, {384, 256, 1.12}, {192, 384, 1.06}, {256, 256, 1.06}, {256, 192, 1.00}, {192, 256, 1.00},
      {256, 128, 0.92}, {128, 256, 0.92}, {128, 128, 0.75}};
  double best = 1e300;
  TileChoice pick = {256, 192};
  for (const auto& c : cand) {
    if (!shared_tiles && c.bm * c.bn > 256 * 192) continue;
    const long tiles = (long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const long waves = (tiles + 255) / 256;
    const double t = (double)waves * c.bm * c.bn / c.eff;
    if (t < best * 0.999) { best = t; pick = {c.bm, c.bn}; }
  }
  return pick;
}

// Column split of a launch that would run as several waves of 256 x 192 tiles:
// the first n1 columns on 256 x 384 tiles filling whole waves, the rest on
// 256 x 192 tiles, when that estimate (the tile efficiencies of choose_tile) is
// lower (the 8192 x 4608 QKV forward: one wave of each instead of three of the
// small tile).  0: no split.
int split_cols(int M, int N) {
  const int64_t tm = (M + 255) / 256;
  const int64_t waves = (tm * ((N + 191) / 192) + 255) / 256;
  if (waves < 2) return 0;
  int best = 0;
  double best_t = (double)waves * 256 * 192;
  for (int n1 = 384; n1 < N; n1 += 384) {
    const int64_t t1 = tm * (n1 / 384), t2 = tm * ((N - n1 + 191) / 192);
    if (t1 % 256 != 0) continue;
    const double t = (double)(t1 / 256) * 256 * 384 / 1.12 + (double)((t2 + 255) / 256) * 256 * 192;
    if (t < best_t * 0.97) { best_t = t; best = n1; }
  }
  return best;
}

template <bool AK, bool BKC, int EPI, typename E>
hipError_t launch_shape(const GemmArgs& g, hipStream_t s, const char** name) {
  // GeLU' with H out stages two strips per wave: only the split tiles hold them
  const TileChoice t = EPI == EPI_DGELU_H ? choose_tile(g.M, g.N, false) : choose_tile(g.M, g.N);
  if constexpr (EPI == EPI_STORE || EPI == EPI_BIAS_GELU || EPI == EPI_DGELU) {
    const int n1 = (t.bm == 256 && t.bn == 192) ? split_cols(g.M, g.N) : 0;
    if (n1 > 0) {
      // columns [0, n1) and [n1, N): every operand and output of the second part
      // starts n1 columns on (B stored [N x K] when BKC: n1 rows on)
      GemmArgs g1 = g, g2 = g;
      g1.N = n1;
      g2.N = g.N - n1;
      g2.B = (const E*)g.B + (BKC ? (int64_t)n1 * g.ldb : (int64_t)n1);
      g2.C = (E*)g.C + n1;
      if (g.C2) g2.C2 = (E*)g.C2 + n1;
      if (g.bias) g2.bias = (const E*)g.bias + n1;
      if (g.aux) g2.aux = (const E*)g.aux + n1;
      static const std::string nm = std::string(kname<T256x384, AK, BKC, EPI, E>()) + "+256x192";
      const char* unused;
      hipError_t e = launch_tile<T256x384, AK, BKC, EPI, E>(g1, s, &unused);
      if (e == hipSuccess) e = launch_tile<T256x192, AK, BKC, EPI, E>(g2, s, &unused);
      *name = nm.c_str();
      return e;
    }
  }
  if constexpr (EPI != EPI_DGELU_H) {
    if (t.bm == 256 && t.bn == 384) return launch_tile<T256x384, AK, BKC, EPI, E>(g, s, name);
    if (t.bm == 384 && t.bn == 256) return launch_tile<T384x256, AK, BKC, EPI, E>(g, s, name);
    if (t.bm == 192 && t.bn == 384) return launch_tile<T192x384, AK, BKC, EPI, E>(g, s, name);
    if (t.bm == 256 && t.bn == 256) return launch_tile<T256x256, AK, BKC, EPI, E>(g, s, name);
  }
  if (t.bm == 256 && t.bn == 192) return launch_tile<T256x192, AK, BKC, EPI, E>(g, s, name);
  if (t.bm == 192 && t.bn == 256) return launch_tile<T192x256, AK, BKC, EPI, E>(g, s, name);
  if (t.bm == 256 && t.bn == 128) return launch_tile<T256x128, AK, BKC, EPI, E>(g, s, name);
  if (t.bm == 128 && t.bn == 256) return launch_tile<T128x256, AK, BKC, EPI, E>(g, s, name);
  return launch_tile<T128x128, AK, BKC, EPI, E>(g, s, name);
}

template <typename E>
hipError_t gemm16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s) {
  LaunchInfo info;
  info.name = "gemm16";
  info.flops = 2.0 * g.M * (double)g.N * g.K;
  // K split of a weight gradient whose tiles fill at most half of the CUs
  GemmArgs gk = g;
  const bool split = epi == EPI_F32 && !a_kcontig && !b_kcontig && g.kpart != nullptr && gemm16_ksplit(g.M, g.N, g.K);
  if (!split) gk.kpart = nullptr;
  const double out_bytes = (epi == EPI_F32 ? 4.0 * (g.accumulate ? 2 : 1) : 2.0) * g.M * (double)g.N +
                           (split ? 4.0 * 4.0 * g.M * (double)g.N : 0.0);   // partial out and in, C again
  info.bytes = 2.0 * ((double)g.M * g.K + (double)g.K * g.N) + out_bytes +
               ((epi == EPI_BIAS_GELU && g.C2) ? 2.0 * g.M * (double)g.N : 0.0) +
               (epi == EPI_DGELU ? 2.0 * g.M * (double)g.N : 0.0) +
               (epi == EPI_DGELU_H ? 4.0 * g.M * (double)g.N : 0.0) +
               (g.colsum ? 4.0 * g.N * (double)gemm16_colsum_rows(g.M, g.N, g.K, split) : 0.0);
  // Instantiated layout / epilogue pairs: forward (NN), data gradient (NT) and
  // weight gradient (TN).
  hipError_t e = hipErrorInvalidValue;
  // column sums: B stored [K x N], fp32 out, a tile that carries them
  if (g.colsum != nullptr && (b_kcontig || epi != EPI_F32 || gemm16_colsum_rows(g.M, g.N, g.K, split) == 0)) return e;
  trace_begin(s);
  if (a_kcontig && !b_kcontig && epi == EPI_STORE) e = launch_shape<true, false, EPI_STORE, E>(gk, s, &info.name);
  else if (a_kcontig && !b_kcontig && epi == EPI_BIAS_GELU)
    e = launch_shape<true, false, EPI_BIAS_GELU, E>(gk, s, &info.name);
  else if (a_kcontig && b_kcontig && epi == EPI_STORE) e = launch_shape<true, true, EPI_STORE, E>(gk, s, &info.name);
  else if (a_kcontig && b_kcontig && epi == EPI_DGELU) e = launch_shape<true, true, EPI_DGELU, E>(gk, s, &info.name);
  else if (a_kcontig && b_kcontig && epi == EPI_DGELU_H && g.C2 != nullptr)
    e = launch_shape<true, true, EPI_DGELU_H, E>(gk, s, &info.name);
  else if (!a_kcontig && !b_kcontig && epi == EPI_F32) e = launch_shape<false, false, EPI_F32, E>(gk, s, &info.name);
  if (split && e == hipSuccess) {
    const int64_t n = (int64_t)g.M * (g.N / 4);
    hipLaunchKernelGGL(kpart_add_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (float*)g.C, g.ldc,
                       (const float*)g.kpart, g.M, g.N);
    e = hipGetLastError();
  }
  trace_end(s, info);
  return e;
}

// Pairing (gemm_pair_kernel) of a data-gradient product g1 (both operands
// K-contiguous) with an independent weight gradient g2 (both operands [K x *],
// fp32 out).  Alone, a g1 of one wave of 256 x 192 tiles (one per CU, the
// tile with the most bytes per FLOP the launcher picks for long contractions
// like the MLP's dH and the out-projection's dX) runs well below the big
// tiles' rate; paired, g1 takes 256 x 384 tiles on at most half of the CUs
// and g2 runs beside it.  Paired when the estimated time, in K steps of a
// 256 x 384 tile, is lower: g1 alone as 256 x 192 tiles costs 0.6 of its
// 256 x 384 time (measured rates), the pair the longer of g1's 256 x 384
// tiles and both products' work spread over all CUs.
constexpr int kPairCUs = 256;

bool pair_plan(const GemmArgs& g1, const GemmArgs& g2, TileChoice* t2) {
  const TileChoice t1 = choose_tile(g1.M, g1.N);
  if (t1.bm != 256 || t1.bn != 192) return false;
  const int64_t small1 = (int64_t)((g1.M + 255) / 256) * ((g1.N + 191) / 192);
  const int64_t n1 = (int64_t)((g1.M + 255) / 256) * ((g1.N + 383) / 384);
  if (small1 > kPairCUs || 2 * n1 > kPairCUs) return false;
  *t2 = choose_tile(g2.M, g2.N);
  if (!((t2->bm == 256 || t2->bm == 192) && t2->bn == 384)) return false;
  if (g2.kpart != nullptr && gemm16_ksplit(g2.M, g2.N, g2.K)) return false;
  const int64_t n2 = (int64_t)((g2.M + t2->bm - 1) / t2->bm) * ((g2.N + 383) / 384);
  if ((n1 + n2) * 512 > (int64_t(1) << 32) - 1) return false;
  const double T1 = (g1.K + KT - 1) / KT;
  const double W2 = (double)n2 * ((g2.K + KT - 1) / KT) * (t2->bm / 256.0);
  const double alone = 0.6 * T1 + W2 / kPairCUs;
  const double paired = std::max(T1, (n1 * T1 + W2) / kPairCUs);
  return paired < 0.97 * alone;
}

template <class C1, int EPI1, class C2, typename E>
std::string pair_name() {
  // the two kernels' names after their "gemm_<type>_" prefix
  const std::string n1 = kname<C1, true, true, EPI1, E>(), n2 = kname<C2, false, false, EPI_F32, E>();
  return std::string("gemm_") + Vec<E>::name + "_pair_" + n1.substr(n1.find('_', 5) + 1) + "+" +
         n2.substr(n2.find('_', 5) + 1);
}

template <class C2, int EPI1, typename E>
hipError_t launch_pair(const GemmArgs& g1_in, const GemmArgs& g2_in, hipStream_t s) {
  GemmArgs g1 = g1_in, g2 = g2_in;
  g2.kpart = nullptr;
  const int tm1 = (g1.M + 255) / 256, tn1 = (g1.N + 383) / 384;
  const int tm2 = (g2.M + C2::BM - 1) / C2::BM, tn2 = (g2.N + C2::BN - 1) / C2::BN;
  g1.group_m = group_for<T256x384, true, true>(tm1);
  g2.group_m = group_for<C2, false, false>(tm2);
  const int n1 = tm1 * tn1;
  hipLaunchKernelGGL((gemm_pair_kernel<T256x384, true, true, EPI1, C2, false, false, EPI_F32, E>),
                     dim3(n1 + tm2 * tn2), dim3(T256x384::NT), 0, s, g1, g2, n1);
  return hipGetLastError();
}

template <typename E>
hipError_t gemm16_pair(const GemmArgs& g1, Epi epi1, const GemmArgs& g2, hipStream_t s) {
  TileChoice t2;
  if (epi1 != EPI_STORE && epi1 != EPI_DGELU) return hipErrorNotSupported;
  if (!pair_plan(g1, g2, &t2)) return hipErrorNotSupported;
  // trace name, e.g. gemm_bf16_pair_nt_dgelu_256x384+tn_f32_256x384
  static const std::string names[2][2] = {
      {pair_name<T256x384, EPI_DGELU, T256x384, E>(), pair_name<T256x384, EPI_STORE, T256x384, E>()},
      {pair_name<T256x384, EPI_DGELU, T192x384, E>(), pair_name<T256x384, EPI_STORE, T192x384, E>()}};
  LaunchInfo info;
  info.name = names[t2.bm == 256 ? 0 : 1][epi1 == EPI_DGELU ? 0 : 1].c_str();
  info.flops = 2.0 * g1.M * (double)g1.N * g1.K + 2.0 * g2.M * (double)g2.N * g2.K;
  info.bytes = 2.0 * ((double)g1.M * g1.K + (double)g1.K * g1.N) + 2.0 * g1.M * (double)g1.N * (epi1 == EPI_DGELU ? 2 : 1) +
               2.0 * ((double)g2.M * g2.K + (double)g2.K * g2.N) + 4.0 * g2.M * (double)g2.N * (g2.accumulate ? 2 : 1) +
               (g2.colsum ? 4.0 * g2.N * (double)gemm16_colsum_rows(g2.M, g2.N, g2.K, false) : 0.0);
  trace_begin(s);
  hipError_t e;
  if (t2.bm == 256) e = epi1 == EPI_DGELU ? launch_pair<T256x384, EPI_DGELU, E>(g1, g2, s) : launch_pair<T256x384, EPI_STORE, E>(g1, g2, s);
  else e = epi1 == EPI_DGELU ? launch_pair<T192x384, EPI_DGELU, E>(g1, g2, s) : launch_pair<T192x384, EPI_STORE, E>(g1, g2, s);
  trace_end(s, info);
  return e;
}

}  // namespace

hipError_t gemm_bf16_pair(const GemmArgs& g1, Epi epi1, const GemmArgs& g2, hipStream_t s) {
  return gemm16_pair<bf16>(g1, epi1, g2, s);
}

hipError_t gemm_f16_pair(const GemmArgs& g1, Epi epi1, const GemmArgs& g2, hipStream_t s) {
  return gemm16_pair<f16>(g1, epi1, g2, s);
}

bool gemm16_pairs(int M1, int N1, int K1, int M2, int N2, int K2, bool split2) {
  GemmArgs g1{}, g2{};
  g1.M = M1; g1.N = N1; g1.K = K1;
  g2.M = M2; g2.N = N2; g2.K = K2;
  float dummy;
  g2.kpart = split2 ? &dummy : nullptr;
  TileChoice t2;
  return pair_plan(g1, g2, &t2);
}

hipError_t gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s) {
  return gemm16<bf16>(g, a_kcontig, b_kcontig, epi, s);
}

hipError_t gemm_f16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, Epi epi, hipStream_t s) {
  return gemm16<f16>(g, a_kcontig, b_kcontig, epi, s);
}

int64_t gemm16_work_items(int64_t M, int64_t N) {
  const TileChoice t = choose_tile((int)M, (int)N);
  int64_t threads = T128x128::NT;
  if (t.bm == 256 && t.bn == 384) threads = T256x384::NT;
  else if (t.bm == 384 && t.bn == 256) threads = T384x256::NT;
  else if (t.bm == 192 && t.bn == 384) threads = T192x384::NT;
  else if (t.bm == 256 && t.bn == 256) threads = T256x256::NT;
  else if (t.bm == 256 && t.bn == 192) threads = T256x192::NT;
  else if (t.bm == 192 && t.bn == 256) threads = T192x256::NT;
  else if (t.bm == 256 && t.bn == 128) threads = T256x128::NT;
  else if (t.bm == 128 && t.bn == 256) threads = T128x256::NT;
  return (M + t.bm - 1) / t.bm * ((N + t.bn - 1) / t.bn) * threads;
}

bool gemm16_ksplit(int M, int N, int K) {
  const TileChoice t = choose_tile(M, N);
  const int64_t tiles = (int64_t)((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  return 2 * tiles <= 256 && K >= 2048;   // at least 32 K steps per half
}

int gemm16_colsum_rows(int M, int N, int K, bool kpart) {
  const TileChoice t = choose_tile(M, N);
  if (t.bm * t.bn >= 256 * 384) return 0;   // that tile does not carry the column sums (Cfg::CSUM)
  return (M + t.bm - 1) / t.bm * (kpart && gemm16_ksplit(M, N, K) ? 2 : 1);
}

}  // namespace tps
