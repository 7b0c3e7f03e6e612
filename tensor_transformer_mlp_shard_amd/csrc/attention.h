// Core attention on a rank's local heads (attention.hip).
#pragma once

#include "common.h"

namespace tps {

// Work-items per workgroup of every attention kernel.
constexpr int kAttnThreads = 256;

// One rank's attention problem.  qkv is [T x 3*Hl*D] bf16 (columns [Q | K | V],
// head-major inside each block), T = B * S tokens in sequences of S.
struct AttnProblem {
  int64_t T;
  int S, Hl, D;
  bool causal;
};

// O [T x Hl*D] bf16 and, when lse is non-null, lse [Hl x T] fp32 (natural log).
hipError_t attention_fwd(const bf16* qkv, bf16* o, float* lse, const AttnProblem& p, hipStream_t s);

// dQKV [T x 3*Hl*D] bf16 from O, lse and dO; ws holds Hl*T floats.
hipError_t attention_bwd(const bf16* qkv, const bf16* o, const float* lse, const bf16* dout, bf16* dqkv,
                         float* ws, const AttnProblem& p, hipStream_t s);

// Algorithmic FLOPs of the forward (2 products of 2*D per allowed query-key pair).
double attention_fwd_flops(const AttnProblem& p);

}  // namespace tps
