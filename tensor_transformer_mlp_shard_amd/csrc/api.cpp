// C ABI of libtpshard.so: argument validation, workspace sizing, launch
// sequencing on the caller's stream, and the optional kernel-timing trace.
// The operations and their sources are documented in include/tpshard.h.
#include "tpshard.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "attention.h"
#include "gemm.h"
#include "side.h"
#include "sp_edge.h"

namespace tps {
namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;      // tokens
constexpr int64_t kMaxFeature = int64_t(1) << 21;  // in/out features (and their shards)
constexpr int64_t kMaxElems = int64_t(1) << 36;
constexpr size_t kAlign = 256;  // workspace sub-buffer alignment

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t elsize(int32_t dtype) { return dtype == TP_FP32 ? 4 : 2; }

// A device buffer an entry point reads or writes, for the overlap check.
struct Buf {
  const void* p;
  size_t bytes;
  Buf(const void* p_, int64_t b) : p(p_), bytes((size_t)b) {}
};

bool overlap(const Buf& a, const Buf& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

int check_dims(std::initializer_list<int64_t> dims) {
  for (int64_t d : dims)
    if (d < 1 || d > kMaxDim) return TP_ERR_DIM;
  return TP_OK;
}

int check_elems(std::initializer_list<std::pair<int64_t, int64_t>> mats) {
  for (const auto& m : mats)
    if (m.first * m.second > kMaxElems) return TP_ERR_DIM;
  return TP_OK;
}

// A launch of `workgroups` workgroups of `threads` work-items each must stay
// within the 32-bit dispatch size (at most 2^32 - 1 work-items in x); sizes the
// other limits admit but one launch cannot cover are rejected up front.
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;
int check_launch(int64_t workgroups, int64_t threads) {
  return workgroups * threads > kMaxWorkItems ? TP_ERR_DIM : TP_OK;
}
// The elementwise passes (bias + GeLU, bias + dropout + residual, dropout
// backward) run one work-item per 8 elements in 256-wide workgroups.
int check_elementwise_launch(int64_t elems) { return check_launch((elems / 8 + 255) / 256, 256); }

// Every GEMM launch (M x N outputs) of an entry point, for the dispatch size.
int check_gemms(int32_t dtype, std::initializer_list<std::pair<int64_t, int64_t>> mn) {
  for (const auto& p : mn) {
    const int64_t w = dtype == TP_FP32 ? gemm_f32_work_items(p.first, p.second) : gemm16_work_items(p.first, p.second);
    if (w > kMaxWorkItems) return TP_ERR_DIM;
  }
  return TP_OK;
}

int check_feature(std::initializer_list<int64_t> dims) {
  for (int64_t d : dims) {
    if (d > kMaxFeature) return TP_ERR_DIM;
    if (d % 8 != 0) return TP_ERR_ALIGNMENT;
  }
  return TP_OK;
}

int check_ptrs_aligned(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && ((uintptr_t)p % 16) != 0) return TP_ERR_ALIGNMENT;
  return TP_OK;
}

int check_nonnull(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p) return TP_ERR_NULLPTR;
  return TP_OK;
}

// No output may overlap an input or another output.
int check_alias(const std::vector<Buf>& ins, const std::vector<Buf>& outs) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Buf& in : ins)
      if (overlap(outs[i], in)) return TP_ERR_ALIAS;
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j])) return TP_ERR_ALIAS;
  }
  return TP_OK;
}

int check_dtype(int32_t dtype) {
  return (dtype == TP_BF16 || dtype == TP_FP32 || dtype == TP_FP16) ? TP_OK : TP_ERR_DTYPE;
}

// The element code of a validated dtype.
Elem elem_of(int32_t dtype) { return dtype == TP_FP32 ? ELEM_F32 : dtype == TP_FP16 ? ELEM_F16 : ELEM_BF16; }

#define TP_TRY(expr)              \
  do {                            \
    const int _st = (expr);       \
    if (_st != TP_OK) return _st; \
  } while (0)

#define HIP_TRY(expr)                              \
  do {                                             \
    if ((expr) != hipSuccess) return TP_ERR_HIP;   \
  } while (0)

hipError_t gemm(int32_t dtype, const GemmArgs& g, bool ak, bool bk, Epi epi, hipStream_t s) {
  if (dtype == TP_FP32) return gemm_f32(g, ak, bk, epi, s);
  return dtype == TP_FP16 ? gemm_f16(g, ak, bk, epi, s) : gemm_bf16(g, ak, bk, epi, s);
}

// g1 and g2 in one launch where the 16-bit GEMM pairs them (see gemm.h);
// hipErrorNotSupported, with nothing launched, where it does not.
hipError_t gemm_pair(int32_t dtype, const GemmArgs& g1, Epi epi1, const GemmArgs& g2, hipStream_t s) {
  if (dtype == TP_FP32) return hipErrorNotSupported;
  return dtype == TP_FP16 ? gemm_f16_pair(g1, epi1, g2, s) : gemm_bf16_pair(g1, epi1, g2, s);
}

// The data gradient g1 and the independent weight gradient g2 of a backward:
// one paired launch where it applies, else one after the other.
hipError_t gemm_dgrad_wgrad(int32_t dtype, const GemmArgs& g1, Epi epi1, const GemmArgs& g2, hipStream_t s) {
  const hipError_t e = gemm_pair(dtype, g1, epi1, g2, s);
  if (e != hipErrorNotSupported) return e;
  const hipError_t e1 = gemm(dtype, g1, true, true, epi1, s);
  if (e1 != hipSuccess) return e1;
  return gemm(dtype, g2, false, false, EPI_F32, s);
}

GemmArgs make_args(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                   void* C, int64_t ldc) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.A = A;
  g.B = B;
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.C = C;
  g.ldc = ldc;
  return g;
}

size_t colsum_ws_bytes(int64_t T, int64_t N) { return round_up((size_t)colsum_chunks(T, N) * (size_t)N * 4); }

// Workspace of a bias gradient db = sum_t dY [N] that goes with a weight
// gradient dW = X^T dY [M x N].  On the 16-bit path the weight-gradient GEMM
// adds dY's columns while dY passes through it (GemmArgs::colsum) and leaves
// one partial row per row of tiles; the fp32 path runs the column-sum pass.
bool db_fused(int32_t dtype, int64_t M, int64_t N) {
  return dtype != TP_FP32 && gemm16_colsum_rows((int)M, (int)N, 1, false) > 0;
}

size_t db_ws_bytes(int32_t dtype, int64_t T, int64_t M, int64_t N) {
  if (!db_fused(dtype, M, N)) return colsum_ws_bytes(T, N);
  return round_up((size_t)gemm16_colsum_rows((int)M, (int)N, (int)T, true) * (size_t)N * 4);
}

// Room for the fp32 partial of a weight gradient [M x N] whose GEMM splits its
// contraction T in two (GemmArgs::kpart), after its bias-gradient partials.
size_t kpart_bytes(int32_t dtype, int64_t T, int64_t M, int64_t N) {
  return dtype != TP_FP32 && gemm16_ksplit((int)M, (int)N, (int)T) ? round_up((size_t)M * (size_t)N * 4) : 0;
}

// The MLP backward's weight-gradient scratch: the bias-gradient partials of
// dB_i [f x h] or dA_i [h x f] (one at a time), then the K-split partial of
// either; mlp_db_part_bytes is the offset of the latter.
size_t mlp_db_part_bytes(int32_t dtype, int64_t T, int64_t h, int64_t f) {
  const size_t c2 = db_ws_bytes(dtype, T, f, h), c1 = db_ws_bytes(dtype, T, h, f);
  return c2 > c1 ? c2 : c1;
}
size_t mlp_wgrad_ws_bytes(int32_t dtype, int64_t T, int64_t h, int64_t f) {
  const size_t k2 = kpart_bytes(dtype, T, f, h), k1 = kpart_bytes(dtype, T, h, f);
  return mlp_db_part_bytes(dtype, T, h, f) + (k2 > k1 ? k2 : k1);
}

// db (+)= sum_t dY after the weight-gradient GEMM g (dW = X^T dY, B = dY) has
// run, with g.colsum = part where db_fused (its partial rows are added here),
// else by the column-sum pass over dY.
hipError_t bias_grad_after_wgrad(const GemmArgs& g, const void* dY, float* db, float* part, int accumulate,
                                 int64_t T, int32_t dtype, hipStream_t s) {
  if (!db_fused(dtype, g.M, g.N)) return colsum(dY, elem_of(dtype), db, part, accumulate, T, g.N, s);
  return sum_partials(part, db, g.N, gemm16_colsum_rows(g.M, g.N, g.K, g.kpart != nullptr), accumulate,
                      "colsum_finalize", s);
}

// Shape checks shared by the attention entry points; fills p on success.
int check_attention(int64_t T, int64_t seq, int64_t heads, int64_t head_dim, int32_t tp_size, int32_t causal,
                    int32_t dtype, AttnProblem& p) {
  if (dtype != TP_BF16) return TP_ERR_DTYPE;  // bf16 only: the attention kernels are MFMA kernels
  if (causal != 0 && causal != 1) return TP_ERR_ARG;
  TP_TRY(check_dims({T, seq, heads}));
  if (head_dim != 64 && head_dim != 128) return TP_ERR_DIM;
  if (T % seq != 0) return TP_ERR_DIM;
  if (tp_size < 1 || heads % tp_size != 0) return TP_ERR_TP_DIVISIBILITY;
  const int64_t hl = heads / tp_size;
  if (3 * hl * head_dim > kMaxFeature) return TP_ERR_DIM;
  // one workgroup of kAttnThreads per 128 queries or per 64 keys of a (sequence, head)
  TP_TRY(check_launch((seq + 63) / 64 * (T / seq) * hl, kAttnThreads));
  p.T = T;
  p.S = (int)seq;
  p.Hl = (int)hl;
  p.D = (int)head_dim;
  p.causal = causal != 0;
  return TP_OK;
}

// ---------------------------------------------------------------- trace
struct TraceAgg {
  std::string name;
  int64_t launches = 0;
  double ms = 0, flops = 0, bytes = 0;
};

struct Trace {
  std::mutex mu;
  bool on = false;
  int max = 0;
  int n = 0;
  std::vector<hipEvent_t> ev;
  std::vector<LaunchInfo> info;
  std::vector<TraceAgg> result;
};

Trace& trace() {
  static Trace t;
  return t;
}

}  // namespace

void trace_begin(hipStream_t stream) {
  Trace& t = trace();
  if (t.on && t.n < t.max) (void)hipEventRecord(t.ev[2 * t.n], stream);
}

void trace_end(hipStream_t stream, const LaunchInfo& info) {
  Trace& t = trace();
  if (t.on && t.n < t.max) {
    (void)hipEventRecord(t.ev[2 * t.n + 1], stream);
    t.info[t.n] = info;
    ++t.n;
  }
}

// Scratch of the allocation-free MLP backward (tp_mlp_shard_bwd_noalloc): a
// static device array, one instance per GPU, loaded with the code object and
// held until the process ends.  Host code never uses its name as an address
// (on the host it names a stand-in object); it uses the device address that
// hipGetSymbolAddress returns for the current GPU, looked up once per device.
constexpr size_t kNoallocScratchBytes = size_t(96) << 20;
__device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of the current GPU's scratch array, or nullptr on a HIP error.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace tps

using namespace tps;

extern "C" {

const char* tp_status_string(int status) {
  switch (status) {
    case TP_OK: return "ok";
    case TP_ERR_NULLPTR: return "a required pointer is NULL";
    case TP_ERR_DIM: return "a dimension is < 1 or too large";
    case TP_ERR_TP_DIVISIBILITY: return "tp_size < 1 or the sharded dimension is not divisible by tp_size";
    case TP_ERR_ALIGNMENT: return "pointer not 16-byte aligned or feature dimension not a multiple of 8";
    case TP_ERR_DTYPE: return "unknown dtype or activation";
    case TP_ERR_ALIAS: return "an output overlaps an input or another output";
    case TP_ERR_WORKSPACE: return "workspace missing or too small";
    case TP_ERR_HIP: return "HIP runtime or kernel launch error";
    case TP_ERR_ARG: return "invalid argument";
    case TP_ERR_SCRATCH: return "the problem needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

size_t tp_workspace_size(int32_t op, int64_t T, int64_t d_in, int64_t d_out, int32_t tp_size, int32_t dtype) {
  if (check_dtype(dtype) != TP_OK || T < 1 || T > kMaxDim) return 0;
  switch (op) {
    case TP_OP_BIAS_GRAD:
      if (d_in < 1 || d_in > kMaxDim) return 0;
      return colsum_ws_bytes(T, d_in);
    case TP_OP_COLUMN_LINEAR_BWD:
      // db_i with dW_i = X^T dY_i [K x N/p], then room for dW_i's K-split partial
      if (tp_size < 1 || d_in < 1 || d_out < 1 || d_in > kMaxDim || d_out > kMaxDim || d_out % tp_size) return 0;
      return db_ws_bytes(dtype, T, d_in, d_out / tp_size) + kpart_bytes(dtype, T, d_in, d_out / tp_size);
    case TP_OP_ROW_LINEAR_BWD:
      // db with dW_i = X_i^T dY [K/p x N], then room for dW_i's K-split partial
      if (tp_size < 1 || d_in < 1 || d_out < 1 || d_in > kMaxDim || d_out > kMaxDim || d_in % tp_size) return 0;
      return db_ws_bytes(dtype, T, d_in / tp_size, d_out) + kpart_bytes(dtype, T, d_in / tp_size, d_out);
    case TP_OP_MLP_SHARD_BWD: {
      // dZ [T x f], then the partials of db2 (with dB_i [f x h]) or db1 (with dA_i [h x f]), one at a time,
      // then room for either weight gradient's K-split partial
      if (tp_size < 1 || d_in < 1 || d_out < 1 || d_in > kMaxDim || d_out > kMaxDim || d_out % tp_size) return 0;
      const int64_t f = d_out / tp_size;
      const size_t dz = round_up((size_t)T * (size_t)f * elsize(dtype));
      return dz + mlp_wgrad_ws_bytes(dtype, T, d_in, f);
    }
    case TP_OP_MLP_SHARD_BWD_RECOMPUTE: {
      // dZ, H and (when Z is not saved) Z [T x f], then the weight-gradient scratch as above
      if (tp_size < 1 || d_in < 1 || d_out < 1 || d_in > kMaxDim || d_out > kMaxDim || d_out % tp_size) return 0;
      const int64_t f = d_out / tp_size;
      const size_t act = round_up((size_t)T * (size_t)f * elsize(dtype));
      return 3 * act + mlp_wgrad_ws_bytes(dtype, T, d_in, f);
    }
    case TP_OP_LAYERNORM_BWD:
      // dgamma and dbeta partial rows of every workgroup (d_in = h)
      if (d_in < 1 || d_in > kMaxFeature) return 0;
      return round_up((size_t)2 * (size_t)layernorm_bwd_chunks(T) * (size_t)d_in * 4);
    case TP_OP_BIAS_DROPOUT_ADD_BWD:
      if (d_in < 1 || d_in > kMaxFeature) return 0;
      return colsum_ws_bytes(T, d_in);
    case TP_OP_ATTENTION_BWD: {
      // d_in = heads, d_out = head_dim: the row-dot Dt [Hl x T] fp32
      if (dtype != TP_BF16 || tp_size < 1 || d_in < 1 || d_in > kMaxDim || d_in % tp_size) return 0;
      if (d_out != 64 && d_out != 128) return 0;
      return round_up((size_t)(d_in / tp_size) * (size_t)T * 4);
    }
    default:
      return 0;
  }
}

int tp_column_linear(const void* X, const void* W_i, const void* b_i, void* Y_i, void* Z_i, int64_t T, int64_t K,
                     int64_t N, int32_t tp_size, int32_t act, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  if (act != TP_ACT_NONE && act != TP_ACT_GELU) return TP_ERR_DTYPE;
  TP_TRY(check_nonnull({X, W_i, Y_i}));
  if (act == TP_ACT_NONE && Z_i) return TP_ERR_ARG;
  TP_TRY(check_dims({T, K, N}));
  if (tp_size < 1 || N % tp_size) return TP_ERR_TP_DIVISIBILITY;
  const int64_t n = N / tp_size;
  TP_TRY(check_feature({K, n}));
  TP_TRY(check_elems({{T, K}, {K, n}, {T, n}}));
  TP_TRY(check_gemms(dtype, {{T, n}}));
  TP_TRY(check_ptrs_aligned({X, W_i, b_i, Y_i, Z_i}));
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X, T * K * es}, {W_i, K * n * es}, {b_i, n * es}},
                     {{Y_i, T * n * es}, {Z_i, Z_i ? T * n * es : 0}}));
  hipStream_t s = (hipStream_t)stream;
  GemmArgs g = make_args(X, K, W_i, n, T, n, K, Y_i, n);
  g.bias = b_i;
  g.C2 = Z_i;
  g.ldc2 = n;
  HIP_TRY(gemm(dtype, g, true, false, act == TP_ACT_GELU ? EPI_BIAS_GELU : EPI_STORE, s));
  return TP_OK;
}

int tp_row_linear(const void* X_i, const void* W_i, const void* b, void* Y_i, int64_t T, int64_t K, int64_t N,
                  int32_t tp_size, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  TP_TRY(check_nonnull({X_i, W_i, Y_i}));
  TP_TRY(check_dims({T, K, N}));
  if (tp_size < 1 || K % tp_size) return TP_ERR_TP_DIVISIBILITY;
  const int64_t k = K / tp_size;
  TP_TRY(check_feature({k, N}));
  TP_TRY(check_elems({{T, k}, {k, N}, {T, N}}));
  TP_TRY(check_gemms(dtype, {{T, N}}));
  TP_TRY(check_ptrs_aligned({X_i, W_i, b, Y_i}));
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X_i, T * k * es}, {W_i, k * N * es}, {b, N * es}}, {{Y_i, T * N * es}}));
  GemmArgs g = make_args(X_i, k, W_i, N, T, N, k, Y_i, N);
  g.bias = b;
  HIP_TRY(gemm(dtype, g, true, false, EPI_STORE, (hipStream_t)stream));
  return TP_OK;
}

int tp_mlp_shard_fwd(const void* X, const void* A_i, const void* b1_i, const void* B_i, void* Z_i, void* H_i,
                     void* Y_i, int64_t T, int64_t h, int64_t F, int32_t tp_size, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  TP_TRY(check_nonnull({X, A_i, B_i, H_i, Y_i}));
  TP_TRY(check_dims({T, h, F}));
  if (tp_size < 1 || F % tp_size) return TP_ERR_TP_DIVISIBILITY;
  const int64_t f = F / tp_size;
  TP_TRY(check_feature({h, f}));
  TP_TRY(check_elems({{T, h}, {h, f}, {T, f}}));
  TP_TRY(check_gemms(dtype, {{T, f}, {T, h}}));
  TP_TRY(check_ptrs_aligned({X, A_i, b1_i, B_i, Z_i, H_i, Y_i}));
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X, T * h * es}, {A_i, h * f * es}, {b1_i, f * es}, {B_i, f * h * es}},
                     {{Z_i, Z_i ? T * f * es : 0}, {H_i, T * f * es}, {Y_i, T * h * es}}));
  hipStream_t s = (hipStream_t)stream;
  GemmArgs g1 = make_args(X, h, A_i, f, T, f, h, H_i, f);
  g1.bias = b1_i;
  g1.C2 = Z_i;
  g1.ldc2 = f;
  HIP_TRY(gemm(dtype, g1, true, false, EPI_BIAS_GELU, s));
  GemmArgs g2 = make_args(H_i, f, B_i, h, T, h, f, Y_i, h);
  HIP_TRY(gemm(dtype, g2, true, false, EPI_STORE, s));
  return TP_OK;
}

// The backward GEMM sequence shared by tp_mlp_shard_bwd and its recompute form.
// H_make non-null (H_i unused): H = GeLU(Z_i) is formed in the dZ GEMM's
// epilogue from the Z it reads anyway, written to H_make, and used from there.
static int mlp_bwd_gemms(const void* X, const void* A_i, const void* B_i, const void* Z_i, const void* H_i, const void* dY,
                  void* dX_i, float* dA_i, float* db1_i, float* dB_i, float* db2, void* dZ, float* part,
                  int32_t accumulate, int64_t T, int64_t h, int64_t f, int32_t dtype, hipStream_t s,
                  void* H_make = nullptr) {
  // room for a K-split weight gradient's partial, after the bias-gradient partials
  float* kp = (float*)((char*)part + mlp_db_part_bytes(dtype, T, h, f));
  // dZ = (dY B_i^T) * GeLU'(Z_i)          [T x f], contraction over h
  GemmArgs g1 = make_args(dY, h, B_i, h, T, f, h, dZ, f);
  g1.aux = Z_i;
  g1.ldaux = f;
  if (H_make) {
    g1.C2 = H_make;
    g1.ldc2 = f;
    H_i = H_make;
  }
  // dB_i = H_i^T dY                       [f x h], contraction over T; db2 = sum_t dY
  GemmArgs g2 = make_args(H_i, f, dY, h, f, h, T, dB_i, h);
  g2.accumulate = accumulate;
  g2.kpart = kp;
  if (db2 && db_fused(dtype, f, h)) g2.colsum = part;
  if (H_make) {
    // H comes out of the dZ GEMM: dB_i after it
    HIP_TRY(gemm(dtype, g1, true, true, EPI_DGELU_H, s));
    HIP_TRY(gemm(dtype, g2, false, false, EPI_F32, s));
  } else {
    HIP_TRY(gemm_dgrad_wgrad(dtype, g1, EPI_DGELU, g2, s));
  }
  if (db2) HIP_TRY(bias_grad_after_wgrad(g2, dY, db2, part, accumulate, T, dtype, s));
  // dA_i = X^T dZ                         [h x f], contraction over T; db1_i = sum_t dZ
  GemmArgs g3 = make_args(X, h, dZ, f, h, f, T, dA_i, f);
  g3.accumulate = accumulate;
  g3.kpart = kp;
  if (db1_i && db_fused(dtype, h, f)) g3.colsum = part;
  HIP_TRY(gemm(dtype, g3, false, false, EPI_F32, s));
  if (db1_i) HIP_TRY(bias_grad_after_wgrad(g3, dZ, db1_i, part, accumulate, T, dtype, s));
  // dX_i = dZ A_i^T                       [T x h], contraction over f
  GemmArgs g4 = make_args(dZ, f, A_i, f, T, h, f, dX_i, h);
  HIP_TRY(gemm(dtype, g4, true, true, EPI_STORE, s));
  return TP_OK;
}

// Argument checks of the MLP backward that do not depend on where its scratch
// lives; on success *need holds the scratch bytes the call uses.
static int mlp_bwd_check(const void* X, const void* A_i, const void* B_i, const void* Z_i, const void* H_i,
                         const void* dY, void* dX_i, float* dA_i, float* db1_i, float* dB_i, float* db2,
                         int32_t accumulate, int64_t T, int64_t h, int64_t F, int32_t tp_size, int32_t dtype,
                         size_t* need) {
  TP_TRY(check_dtype(dtype));
  if (accumulate != 0 && accumulate != 1) return TP_ERR_ARG;
  TP_TRY(check_nonnull({X, A_i, B_i, Z_i, H_i, dY, dX_i, dA_i, dB_i}));
  TP_TRY(check_dims({T, h, F}));
  if (tp_size < 1 || F % tp_size) return TP_ERR_TP_DIVISIBILITY;
  const int64_t f = F / tp_size;
  TP_TRY(check_feature({h, f}));
  TP_TRY(check_elems({{T, h}, {h, f}, {T, f}}));
  TP_TRY(check_gemms(dtype, {{T, f}, {f, h}, {h, f}, {T, h}}));
  TP_TRY(check_ptrs_aligned({X, A_i, B_i, Z_i, H_i, dY, dX_i, dA_i, db1_i, dB_i, db2}));
  *need = tp_workspace_size(TP_OP_MLP_SHARD_BWD, T, h, F, tp_size, dtype);
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X, T * h * es}, {A_i, h * f * es}, {B_i, f * h * es}, {Z_i, T * f * es},
                      {H_i, T * f * es}, {dY, T * h * es}},
                     {{dX_i, T * h * es}, {dA_i, h * f * 4}, {db1_i, db1_i ? f * 4 : 0}, {dB_i, f * h * 4},
                      {db2, db2 ? h * 4 : 0}}));
  return TP_OK;
}

// The MLP backward on validated arguments, with its scratch (dZ, then the
// column-sum partials) at `ws`.
static int mlp_bwd_run(const void* X, const void* A_i, const void* B_i, const void* Z_i, const void* H_i,
                       const void* dY, void* dX_i, float* dA_i, float* db1_i, float* dB_i, float* db2, char* ws,
                       int32_t accumulate, int64_t T, int64_t h, int64_t F, int32_t tp_size, int32_t dtype,
                       hipStream_t s) {
  const int64_t f = F / tp_size;
  float* part = (float*)(ws + round_up((size_t)T * (size_t)f * elsize(dtype)));
  return mlp_bwd_gemms(X, A_i, B_i, Z_i, H_i, dY, dX_i, dA_i, db1_i, dB_i, db2, ws, part, accumulate, T, h, f,
                       dtype, s);
}

int tp_mlp_shard_bwd(const void* X, const void* A_i, const void* B_i, const void* Z_i, const void* H_i,
                     const void* dY, void* dX_i, float* dA_i, float* db1_i, float* dB_i, float* db2,
                     void* workspace, size_t workspace_bytes, int32_t accumulate, int64_t T, int64_t h, int64_t F,
                     int32_t tp_size, int32_t dtype, void* stream) {
  size_t need = 0;
  TP_TRY(mlp_bwd_check(X, A_i, B_i, Z_i, H_i, dY, dX_i, dA_i, db1_i, dB_i, db2, accumulate, T, h, F, tp_size, dtype,
                       &need));
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  TP_TRY(check_ptrs_aligned({workspace}));
  const int64_t es = elsize(dtype);
  const int64_t f = F / tp_size;
  TP_TRY(check_alias({{X, T * h * es}, {A_i, h * f * es}, {B_i, f * h * es}, {Z_i, T * f * es},
                      {H_i, T * f * es}, {dY, T * h * es}, {dX_i, T * h * es}, {dA_i, h * f * 4},
                      {db1_i, db1_i ? f * 4 : 0}, {dB_i, f * h * 4}, {db2, db2 ? h * 4 : 0}},
                     {{workspace, (int64_t)need}}));
  return mlp_bwd_run(X, A_i, B_i, Z_i, H_i, dY, dX_i, dA_i, db1_i, dB_i, db2, (char*)workspace, accumulate, T, h, F,
                     tp_size, dtype, (hipStream_t)stream);
}

size_t tp_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

int tp_mlp_shard_bwd_noalloc(const void* X, const void* A_i, const void* B_i, const void* Z_i, const void* H_i,
                             const void* dY, void* dX_i, float* dA_i, float* db1_i, float* dB_i, float* db2,
                             int32_t accumulate, int64_t T, int64_t h, int64_t F, int32_t tp_size, int32_t dtype,
                             void* stream) {
  size_t need = 0;
  TP_TRY(mlp_bwd_check(X, A_i, B_i, Z_i, H_i, dY, dX_i, dA_i, db1_i, dB_i, db2, accumulate, T, h, F, tp_size, dtype,
                       &need));
  if (need > kNoallocScratchBytes) return TP_ERR_SCRATCH;
  // Every scratch byte the backward reads (dZ, the column-sum partials) is
  // written earlier in the same call, so nothing is cleared.
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return TP_ERR_HIP;
  return mlp_bwd_run(X, A_i, B_i, Z_i, H_i, dY, dX_i, dA_i, db1_i, dB_i, db2, (char*)ws, accumulate, T, h, F,
                     tp_size, dtype, (hipStream_t)stream);
}

int tp_mlp_shard_bwd_recompute(const void* X, const void* A_i, const void* b1_i, const void* B_i, const void* Z_i,
                               const void* dY, void* dX_i, float* dA_i, float* db1_i, float* dB_i, float* db2,
                               void* workspace, size_t workspace_bytes, int32_t accumulate, int64_t T, int64_t h,
                               int64_t F, int32_t tp_size, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  if (accumulate != 0 && accumulate != 1) return TP_ERR_ARG;
  TP_TRY(check_nonnull({X, A_i, B_i, dY, dX_i, dA_i, dB_i}));
  TP_TRY(check_dims({T, h, F}));
  if (tp_size < 1 || F % tp_size) return TP_ERR_TP_DIVISIBILITY;
  const int64_t f = F / tp_size;
  TP_TRY(check_feature({h, f}));
  TP_TRY(check_elems({{T, h}, {h, f}, {T, f}}));
  TP_TRY(check_gemms(dtype, {{T, f}, {f, h}, {h, f}, {T, h}}));
  TP_TRY(check_ptrs_aligned({X, A_i, b1_i, B_i, Z_i, dY, dX_i, dA_i, db1_i, dB_i, db2, workspace}));
  const size_t need = tp_workspace_size(TP_OP_MLP_SHARD_BWD_RECOMPUTE, T, h, F, tp_size, dtype);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X, T * h * es}, {A_i, h * f * es}, {b1_i, b1_i ? f * es : 0}, {B_i, f * h * es},
                      {Z_i, Z_i ? T * f * es : 0}, {dY, T * h * es}},
                     {{dX_i, T * h * es}, {dA_i, h * f * 4}, {db1_i, db1_i ? f * 4 : 0}, {dB_i, f * h * 4},
                      {db2, db2 ? h * 4 : 0}, {workspace, (int64_t)need}}));
  hipStream_t s = (hipStream_t)stream;
  const size_t act = round_up((size_t)T * (size_t)f * es);
  char* ws = (char*)workspace;
  void* dZ = ws;
  void* H = ws + act;
  const void* Z = Z_i;
  if (Z_i == nullptr) {
    // nothing saved: Z and H again from the forward's fused GEMM (same kernel, same inputs)
    void* Zw = ws + 2 * act;
    GemmArgs g = make_args(X, h, A_i, f, T, f, h, H, f);
    g.bias = b1_i;
    g.C2 = Zw;
    g.ldc2 = f;
    HIP_TRY(gemm(dtype, g, true, false, EPI_BIAS_GELU, s));
    Z = Zw;
  }
  float* part = (float*)(ws + 3 * act);
  // Z saved (it already holds the bias): H = GeLU(Z) comes out of the dZ GEMM's
  // epilogue, which reads Z anyway; recomputed from X: H is the fc1 output
  return mlp_bwd_gemms(X, A_i, B_i, Z, H, dY, dX_i, dA_i, db1_i, dB_i, db2, dZ, part, accumulate, T, h, f, dtype,
                       s, Z_i != nullptr ? H : nullptr);
}

int tp_column_linear_bwd(const void* X, const void* W_i, const void* dY_i, void* dX_partial, float* dW_i,
                         float* db_i, void* workspace, size_t workspace_bytes, int32_t accumulate, int64_t T,
                         int64_t K, int64_t N, int32_t tp_size, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  if (accumulate != 0 && accumulate != 1) return TP_ERR_ARG;
  TP_TRY(check_nonnull({X, W_i, dY_i, dX_partial, dW_i}));
  TP_TRY(check_dims({T, K, N}));
  if (tp_size < 1 || N % tp_size) return TP_ERR_TP_DIVISIBILITY;
  const int64_t n = N / tp_size;
  TP_TRY(check_feature({K, n}));
  TP_TRY(check_elems({{T, K}, {K, n}, {T, n}}));
  TP_TRY(check_gemms(dtype, {{T, K}, {K, n}}));
  TP_TRY(check_ptrs_aligned({X, W_i, dY_i, dX_partial, dW_i, db_i, workspace}));
  const size_t need = db_i ? tp_workspace_size(TP_OP_COLUMN_LINEAR_BWD, T, K, N, tp_size, dtype) : 0;
  if (db_i && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  // dW_i's K split where the workspace has room for its partial (a caller without db may pass none)
  const size_t dbb = db_ws_bytes(dtype, T, K, n), kpb = kpart_bytes(dtype, T, K, n);
  const bool use_kp = kpb && workspace && workspace_bytes >= dbb + kpb;
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X, T * K * es}, {W_i, K * n * es}, {dY_i, T * n * es}},
                     {{dX_partial, T * K * es}, {dW_i, K * n * 4}, {db_i, db_i ? n * 4 : 0},
                      {workspace, (int64_t)(use_kp ? dbb + kpb : need)}}));
  hipStream_t s = (hipStream_t)stream;
  // dX = dY_i W_i^T  [T x K], contraction over n
  GemmArgs g1 = make_args(dY_i, n, W_i, n, T, K, n, dX_partial, K);
  // dW_i = X^T dY_i  [K x n], contraction over T; db_i = sum_t dY_i
  GemmArgs g2 = make_args(X, K, dY_i, n, K, n, T, dW_i, n);
  g2.accumulate = accumulate;
  if (db_i && db_fused(dtype, K, n)) g2.colsum = (float*)workspace;
  if (use_kp) g2.kpart = (float*)((char*)workspace + dbb);
  HIP_TRY(gemm_dgrad_wgrad(dtype, g1, EPI_STORE, g2, s));
  if (db_i) HIP_TRY(bias_grad_after_wgrad(g2, dY_i, db_i, (float*)workspace, accumulate, T, dtype, s));
  return TP_OK;
}

int tp_row_linear_bwd(const void* X_i, const void* W_i, const void* dY, void* dX_i, float* dW_i, float* db,
                      void* workspace, size_t workspace_bytes, int32_t accumulate, int64_t T, int64_t K, int64_t N,
                      int32_t tp_size, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  if (accumulate != 0 && accumulate != 1) return TP_ERR_ARG;
  TP_TRY(check_nonnull({X_i, W_i, dY, dX_i, dW_i}));
  TP_TRY(check_dims({T, K, N}));
  if (tp_size < 1 || K % tp_size) return TP_ERR_TP_DIVISIBILITY;
  const int64_t k = K / tp_size;
  TP_TRY(check_feature({k, N}));
  TP_TRY(check_elems({{T, k}, {k, N}, {T, N}}));
  TP_TRY(check_gemms(dtype, {{T, k}, {k, N}}));
  TP_TRY(check_ptrs_aligned({X_i, W_i, dY, dX_i, dW_i, db, workspace}));
  const size_t need = db ? tp_workspace_size(TP_OP_ROW_LINEAR_BWD, T, K, N, tp_size, dtype) : 0;
  if (db && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  // dW_i's K split where the workspace has room for its partial (a caller without db may pass none)
  const size_t dbb = db_ws_bytes(dtype, T, k, N), kpb = kpart_bytes(dtype, T, k, N);
  const bool use_kp = kpb && workspace && workspace_bytes >= dbb + kpb;
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X_i, T * k * es}, {W_i, k * N * es}, {dY, T * N * es}},
                     {{dX_i, T * k * es}, {dW_i, k * N * 4}, {db, db ? N * 4 : 0},
                      {workspace, (int64_t)(use_kp ? dbb + kpb : need)}}));
  hipStream_t s = (hipStream_t)stream;
  // dX_i = dY W_i^T  [T x k], contraction over N
  GemmArgs g1 = make_args(dY, N, W_i, N, T, k, N, dX_i, k);
  // dW_i = X_i^T dY  [k x N], contraction over T; db = sum_t dY
  GemmArgs g2 = make_args(X_i, k, dY, N, k, N, T, dW_i, N);
  g2.accumulate = accumulate;
  if (db && db_fused(dtype, k, N)) g2.colsum = (float*)workspace;
  if (use_kp) g2.kpart = (float*)((char*)workspace + dbb);
  HIP_TRY(gemm_dgrad_wgrad(dtype, g1, EPI_STORE, g2, s));
  if (db) HIP_TRY(bias_grad_after_wgrad(g2, dY, db, (float*)workspace, accumulate, T, dtype, s));
  return TP_OK;
}

int tp_bias_grad(const void* dY, float* db, void* workspace, size_t workspace_bytes, int32_t accumulate, int64_t T,
                 int64_t N, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  if (accumulate != 0 && accumulate != 1) return TP_ERR_ARG;
  TP_TRY(check_nonnull({dY, db}));
  TP_TRY(check_dims({T, N}));
  TP_TRY(check_feature({N}));
  TP_TRY(check_elems({{T, N}}));
  TP_TRY(check_ptrs_aligned({dY, db, workspace}));
  const size_t need = tp_workspace_size(TP_OP_BIAS_GRAD, T, N, 0, 1, dtype);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  TP_TRY(check_alias({{dY, T * N * elsize(dtype)}}, {{db, N * 4}, {workspace, (int64_t)need}}));
  HIP_TRY(colsum(dY, elem_of(dtype), db, (float*)workspace, accumulate, T, N, (hipStream_t)stream));
  return TP_OK;
}

int tp_bias_gelu(const void* Z, const void* b, void* H, int64_t T, int64_t N, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  TP_TRY(check_nonnull({Z, H}));
  TP_TRY(check_dims({T, N}));
  TP_TRY(check_feature({N}));
  TP_TRY(check_elems({{T, N}}));
  TP_TRY(check_elementwise_launch(T * N));
  TP_TRY(check_ptrs_aligned({Z, b, H}));
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{Z, T * N * es}, {b, N * es}}, {{H, T * N * es}}));
  HIP_TRY(bias_gelu(Z, b, H, elem_of(dtype), T, N, (hipStream_t)stream));
  return TP_OK;
}

// ---------------------------------------------------------------- core attention
int tp_attention_fwd(const void* QKV_i, void* O_i, float* lse, int64_t T, int64_t seq, int64_t heads,
                     int64_t head_dim, int32_t tp_size, int32_t causal, int32_t dtype, void* stream) {
  AttnProblem p;
  TP_TRY(check_attention(T, seq, heads, head_dim, tp_size, causal, dtype, p));
  TP_TRY(check_nonnull({QKV_i, O_i}));
  TP_TRY(check_ptrs_aligned({QKV_i, O_i, lse}));
  const int64_t w = (int64_t)p.Hl * p.D;
  TP_TRY(check_alias({{QKV_i, T * 3 * w * 2}}, {{O_i, T * w * 2}, {lse, lse ? T * p.Hl * 4 : 0}}));
  HIP_TRY(attention_fwd((const bf16*)QKV_i, (bf16*)O_i, lse, p, (hipStream_t)stream));
  return TP_OK;
}

int tp_attention_bwd(const void* QKV_i, const void* O_i, const float* lse, const void* dO_i, void* dQKV_i,
                     void* workspace, size_t workspace_bytes, int64_t T, int64_t seq, int64_t heads,
                     int64_t head_dim, int32_t tp_size, int32_t causal, int32_t dtype, void* stream) {
  AttnProblem p;
  TP_TRY(check_attention(T, seq, heads, head_dim, tp_size, causal, dtype, p));
  TP_TRY(check_nonnull({QKV_i, O_i, lse, dO_i, dQKV_i}));
  TP_TRY(check_ptrs_aligned({QKV_i, O_i, lse, dO_i, dQKV_i, workspace}));
  const size_t need = tp_workspace_size(TP_OP_ATTENTION_BWD, T, heads, head_dim, tp_size, dtype);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  const int64_t w = (int64_t)p.Hl * p.D;
  TP_TRY(check_alias({{QKV_i, T * 3 * w * 2}, {O_i, T * w * 2}, {lse, T * p.Hl * 4}, {dO_i, T * w * 2}},
                     {{dQKV_i, T * 3 * w * 2}, {workspace, (int64_t)need}}));
  HIP_TRY(attention_bwd((const bf16*)QKV_i, (const bf16*)O_i, lse, (const bf16*)dO_i, (bf16*)dQKV_i,
                        (float*)workspace, p, (hipStream_t)stream));
  return TP_OK;
}

// ---------------------------------------------------------------- sequence-parallel edge steps
static int check_rows_h(int64_t rows, int64_t h) {
  TP_TRY(check_dims({rows, h}));
  TP_TRY(check_feature({h}));
  TP_TRY(check_elems({{rows, h}}));
  return TP_OK;
}

static int dropout_params(double p_drop, uint64_t offset, uint64_t& threshold, float& scale) {
  if (!(p_drop >= 0.0 && p_drop < 1.0)) return TP_ERR_ARG;
  if (offset % 8 != 0) return TP_ERR_ARG;
  threshold = (uint64_t)std::floor((1.0 - p_drop) * 4294967296.0);
  scale = (float)(1.0 / (1.0 - p_drop));
  return TP_OK;
}

int tp_layernorm_fwd(const void* X, const void* gamma, const void* beta, void* Y, float* mean, float* rstd,
                     int64_t rows, int64_t h, float eps, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  TP_TRY(check_nonnull({X, gamma, Y}));
  if ((mean == nullptr) != (rstd == nullptr)) return TP_ERR_ARG;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return TP_ERR_ARG;
  TP_TRY(check_rows_h(rows, h));
  TP_TRY(check_launch(rows, layernorm_fwd_threads()));   // one workgroup per row
  TP_TRY(check_ptrs_aligned({X, gamma, beta, Y, mean, rstd}));
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X, rows * h * es}, {gamma, h * es}, {beta, beta ? h * es : 0}},
                     {{Y, rows * h * es}, {mean, mean ? rows * 4 : 0}, {rstd, rstd ? rows * 4 : 0}}));
  HIP_TRY(layernorm_fwd(X, gamma, beta, Y, mean, rstd, rows, h, eps, elem_of(dtype), (hipStream_t)stream));
  return TP_OK;
}

int tp_layernorm_bwd(const void* X, const void* gamma, const float* mean, const float* rstd, const void* dY, void* dX,
                     float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes, int32_t accumulate,
                     int64_t rows, int64_t h, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  if (accumulate != 0 && accumulate != 1) return TP_ERR_ARG;
  TP_TRY(check_nonnull({X, gamma, mean, rstd, dY, dX, dgamma}));
  TP_TRY(check_rows_h(rows, h));
  TP_TRY(check_ptrs_aligned({X, gamma, mean, rstd, dY, dX, dgamma, dbeta, workspace}));
  const size_t need = tp_workspace_size(TP_OP_LAYERNORM_BWD, rows, h, 0, 1, dtype);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{X, rows * h * es}, {gamma, h * es}, {mean, rows * 4}, {rstd, rows * 4}, {dY, rows * h * es}},
                     {{dX, rows * h * es}, {dgamma, h * 4}, {dbeta, dbeta ? h * 4 : 0},
                      {workspace, (int64_t)need}}));
  HIP_TRY(layernorm_bwd(X, gamma, mean, rstd, dY, dX, dgamma, dbeta, (float*)workspace, accumulate, rows, h,
                        elem_of(dtype), (hipStream_t)stream));
  return TP_OK;
}

int tp_bias_dropout_add_fwd(const void* Y, const void* b, const void* residual, void* out, int64_t rows, int64_t h,
                            double p_drop, uint64_t seed, uint64_t offset, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  TP_TRY(check_nonnull({Y, residual, out}));
  TP_TRY(check_rows_h(rows, h));
  uint64_t thr;
  float scale;
  TP_TRY(dropout_params(p_drop, offset, thr, scale));
  TP_TRY(check_elementwise_launch(rows * h));
  TP_TRY(check_ptrs_aligned({Y, b, residual, out}));
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{Y, rows * h * es}, {b, b ? h * es : 0}, {residual, rows * h * es}}, {{out, rows * h * es}}));
  HIP_TRY(bias_dropout_add_fwd(Y, b, residual, out, rows, h, thr, scale, seed, offset, elem_of(dtype),
                               (hipStream_t)stream));
  return TP_OK;
}

int tp_bias_dropout_add_bwd(const void* dOut, void* dY, float* db, void* workspace, size_t workspace_bytes,
                            int32_t accumulate, int64_t rows, int64_t h, double p_drop, uint64_t seed,
                            uint64_t offset, int32_t dtype, void* stream) {
  TP_TRY(check_dtype(dtype));
  if (accumulate != 0 && accumulate != 1) return TP_ERR_ARG;
  TP_TRY(check_nonnull({dOut, dY}));
  TP_TRY(check_rows_h(rows, h));
  uint64_t thr;
  float scale;
  TP_TRY(dropout_params(p_drop, offset, thr, scale));
  TP_TRY(check_elementwise_launch(rows * h));
  TP_TRY(check_ptrs_aligned({dOut, dY, db, workspace}));
  const size_t need = db ? tp_workspace_size(TP_OP_BIAS_DROPOUT_ADD_BWD, rows, h, 0, 1, dtype) : 0;
  if (db && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  const int64_t es = elsize(dtype);
  TP_TRY(check_alias({{dOut, rows * h * es}},
                     {{dY, rows * h * es}, {db, db ? h * 4 : 0}, {workspace, db ? (int64_t)need : 0}}));
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(dropout_bwd(dOut, dY, rows, h, thr, scale, seed, offset, elem_of(dtype), s));
  if (db) HIP_TRY(colsum(dY, elem_of(dtype), db, (float*)workspace, accumulate, rows, h, s));
  return TP_OK;
}

// ---------------------------------------------------------------- loss scaling
int tp_unscale_check_finite(float* grads, int64_t n, float inv_scale, int32_t* found_nonfinite, void* stream) {
  TP_TRY(check_nonnull({grads, found_nonfinite}));
  if (n < 1 || n > kMaxElems) return TP_ERR_DIM;
  if (!(inv_scale > 0.0f) || !std::isfinite(inv_scale)) return TP_ERR_ARG;
  TP_TRY(check_ptrs_aligned({grads}));
  if ((uintptr_t)found_nonfinite % 4 != 0) return TP_ERR_ALIGNMENT;
  TP_TRY(check_alias({{grads, n * 4}}, {{found_nonfinite, 4}}));
  HIP_TRY(unscale_check(grads, n, inv_scale, (int*)found_nonfinite, (hipStream_t)stream));
  return TP_OK;
}

// ---------------------------------------------------------------- probe
int tp_mfma_probe(int32_t blocks, int32_t iters, float* sink, unsigned long long* ticks, void* stream) {
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 24)) return TP_ERR_ARG;
  if (!sink || !ticks) return TP_ERR_NULLPTR;
  if ((uintptr_t)ticks % 8 != 0 || (uintptr_t)sink % 4 != 0) return TP_ERR_ALIGNMENT;
  HIP_TRY(mfma_probe(blocks, iters, sink, ticks, (hipStream_t)stream));
  return TP_OK;
}

int tp_wall_clock_rate_khz(int32_t* khz) {
  if (!khz) return TP_ERR_NULLPTR;
  int dev = 0, rate = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TP_ERR_HIP;
  if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate <= 0) return TP_ERR_HIP;
  *khz = rate;
  return TP_OK;
}

// ---------------------------------------------------------------- trace
int tp_trace_start(int32_t max_launches) {
  Trace& t = trace();
  std::lock_guard<std::mutex> lock(t.mu);
  if (max_launches < 1) return TP_ERR_ARG;
  if ((int)t.ev.size() < 2 * max_launches) {
    const size_t old = t.ev.size();
    t.ev.resize(2 * (size_t)max_launches);
    for (size_t i = old; i < t.ev.size(); ++i)
      if (hipEventCreate(&t.ev[i]) != hipSuccess) {
        t.ev.resize(i);
        return TP_ERR_HIP;
      }
  }
  t.info.assign(max_launches, LaunchInfo{nullptr, 0, 0});
  t.max = max_launches;
  t.n = 0;
  t.on = true;
  return TP_OK;
}

int tp_trace_stop(void) {
  Trace& t = trace();
  std::lock_guard<std::mutex> lock(t.mu);
  if (!t.on) return TP_ERR_ARG;
  t.on = false;
  t.result.clear();
  if (t.n == 0) return TP_OK;
  if (hipEventSynchronize(t.ev[2 * t.n - 1]) != hipSuccess) return TP_ERR_HIP;
  std::map<std::string, size_t> index;
  for (int i = 0; i < t.n; ++i) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) return TP_ERR_HIP;
    const std::string name = t.info[i].name ? t.info[i].name : "?";
    auto it = index.find(name);
    if (it == index.end()) {
      it = index.emplace(name, t.result.size()).first;
      t.result.push_back(TraceAgg{name});
    }
    TraceAgg& a = t.result[it->second];
    a.launches += 1;
    a.ms += ms;
    a.flops += t.info[i].flops;
    a.bytes += t.info[i].bytes;
  }
  return TP_OK;
}

int tp_trace_num_kernels(void) {
  Trace& t = trace();
  std::lock_guard<std::mutex> lock(t.mu);
  return (int)t.result.size();
}

int tp_trace_kernel(int32_t idx, char* name, size_t name_len, int64_t* launches, double* total_ms, double* flops,
                    double* bytes) {
  Trace& t = trace();
  std::lock_guard<std::mutex> lock(t.mu);
  if (idx < 0 || idx >= (int)t.result.size()) return TP_ERR_ARG;
  const TraceAgg& a = t.result[idx];
  if (name && name_len) {
    std::strncpy(name, a.name.c_str(), name_len - 1);
    name[name_len - 1] = '\0';
  }
  if (launches) *launches = a.launches;
  if (total_ms) *total_ms = a.ms;
  if (flops) *flops = a.flops;
  if (bytes) *bytes = a.bytes;
  return TP_OK;
}

}  // extern "C"
