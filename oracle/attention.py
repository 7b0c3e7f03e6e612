"""fp64 CPU oracle for core attention on one rank's local heads.

TEST INFRASTRUCTURE ONLY. This module is imported by the test suite, by the
package smoke check and by the benchmark's CPU-baseline leg. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
it imports nothing from the product path.

Sources (the web pages this method is described on):

* [TUT]  "Megatron-LM：NVIDIA 的大规模并行训练方案", section "Megatron-LM 核心
  架构 / 张量并行原理": the Q, K and V projections are column-parallel and the
  output projection row-parallel, so each rank holds whole heads and runs
  attention on them with no communication between the two.  Section
  "环境搭建与安装 / 依赖项" and "最佳实践与调优建议" (FlashAttention): the
  attention kernel can be replaced by an IO-aware exact one; "混合精度" in the
  same section: query-key layer scaling guards fp16 scores against overflow
  (a rescaling that cancels inside the softmax; it does not change the result).
* [INTRO] "课程导入", section 1.3.1: the Transformer block's self-attention is
  multi-head attention.
* [BASICS] "分布式训练基础…", section 2.2, "案例拆解：175B 的张量并行": the QKV
  matrix 12288 x 36864 in 8 shards of 12288 x 4608 (so each rank's shard holds
  a third of its width for each of Q, K and V).

Readings taken where the pages are silent:

* Scaled dot-product attention per head with the causal mask of a GPT
  decoder: O = softmax(Q K^T / sqrt(d) + M) V, M[i, j] = -inf for j > i.
* The rank's QKV shard row t is [Q | K | V], each block head-major
  ([head][d]); the attention output O_i row t is [head][d], the layout the
  output projection's row shard reads.
* Tokens are sequences of length S packed back to back: T = B * S; attention
  never crosses a sequence boundary.
* No attention dropout (the pages give no rate; the GPU path is deterministic).
* The log-sum-exp saved for the backward is natural-log: lse[h, t] =
  log sum_j exp(s_tj) over the allowed keys, s = q.k / sqrt(d).
* The backward is the chain rule of the forward, pinned by finite
  differences in the tests.

Everything is computed in float64 with no intermediate rounding; matrix
products are numpy float64 matmuls used as a library primitive.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "split_qkv",
    "merge_heads",
    "attention_head_fwd",
    "attention_head_bwd",
    "core_attention_fwd",
    "core_attention_bwd",
]


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def split_qkv(QKV, heads_local: int, d: int):
    """[T x 3*Hl*d] -> Q, K, V, each [Hl, T, d].  Column block 0 of the shard is
    Q, block 1 is K, block 2 is V; inside a block head h owns columns
    h*d .. h*d + d - 1."""
    QKV = _f64(QKV)
    T, W = QKV.shape
    if W != 3 * heads_local * d:
        raise ValueError(f"QKV width {W} != 3 * {heads_local} * {d}")
    blocks = QKV.reshape(T, 3, heads_local, d)
    Q = np.ascontiguousarray(blocks[:, 0].transpose(1, 0, 2))
    K = np.ascontiguousarray(blocks[:, 1].transpose(1, 0, 2))
    V = np.ascontiguousarray(blocks[:, 2].transpose(1, 0, 2))
    return Q, K, V


def merge_heads(X) -> np.ndarray:
    """[Hl, T, d] -> [T x Hl*d] (head-major columns)."""
    X = _f64(X)
    Hl, T, d = X.shape
    return np.ascontiguousarray(X.transpose(1, 0, 2).reshape(T, Hl * d))


def _scores(q, k, causal: bool):
    S, d = q.shape
    s = (q @ k.T) / math.sqrt(d)
    if causal:
        i = np.arange(S)[:, None]
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j > i, -np.inf, s)
    return s


def attention_head_fwd(q, k, v, causal: bool = True):
    """One head of one sequence: q, k, v [S x d].  Returns (O [S x d], lse [S],
    P [S x S]) with P = softmax over the allowed keys of q.k / sqrt(d)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = _scores(q, k, causal)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    P = e / l
    O = P @ v
    lse = m[:, 0] + np.log(l[:, 0])
    return O, lse, P


def attention_head_bwd(q, k, v, dO, causal: bool = True, o=None, return_ds: bool = False):
    """Gradients of sum(dO * O) for one head of one sequence.

    With P the forward's probabilities and s the scaled scores:
      dV = P^T dO;  dP = dO V^T;  ds = P * (dP - D);  D = rowsum(P * dP);
      dQ = ds K / sqrt(d);  dK = ds^T Q / sqrt(d).
    D equals rowsum(dO * O) (the softmax Jacobian).  The IO-aware backward
    takes D from the output the forward stored; passing that output as `o`
    gives the gradients of that formulation, D = rowsum(dO * o) (equal to the
    default when `o` is the exact output).  return_ds: also return ds [S x S]."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    d = q.shape[1]
    _, _, P = attention_head_fwd(q, k, v, causal)
    dV = P.T @ dO
    dP = dO @ v.T
    D = np.sum(P * dP, axis=1, keepdims=True) if o is None else np.sum(dO * _f64(o), axis=1, keepdims=True)
    ds = P * (dP - D)
    dQ = (ds @ k) / math.sqrt(d)
    dK = (ds.T @ q) / math.sqrt(d)
    return (dQ, dK, dV, ds) if return_ds else (dQ, dK, dV)


def core_attention_fwd(QKV, seq: int, heads_local: int, d: int, causal: bool = True):
    """Attention on every local head of every sequence of a rank's QKV shard.

    QKV [T x 3*Hl*d] with T = B * seq.  Returns O [T x Hl*d] and lse [Hl x T]."""
    Q, K, V = split_qkv(QKV, heads_local, d)
    Hl, T, _ = Q.shape
    if seq < 1 or T % seq != 0:
        raise ValueError(f"T={T} is not a whole number of sequences of length {seq}")
    O = np.zeros((Hl, T, d))
    lse = np.zeros((Hl, T))
    for h in range(Hl):
        for b0 in range(0, T, seq):
            sl = slice(b0, b0 + seq)
            O[h, sl], lse[h, sl], _ = attention_head_fwd(Q[h, sl], K[h, sl], V[h, sl], causal)
    return merge_heads(O), lse


def core_attention_bwd(QKV, dO, seq: int, heads_local: int, d: int, causal: bool = True, O=None):
    """dQKV [T x 3*Hl*d] (same [Q | K | V] layout as the input) of sum(dO * O).
    O [T x Hl*d], if given, is the stored forward output the D term is taken
    from (see attention_head_bwd)."""
    Q, K, V = split_qkv(QKV, heads_local, d)
    Hl, T, _ = Q.shape
    dO3 = _f64(dO).reshape(T, Hl, d).transpose(1, 0, 2)
    O3 = None if O is None else _f64(O).reshape(T, Hl, d).transpose(1, 0, 2)
    if seq < 1 or T % seq != 0:
        raise ValueError(f"T={T} is not a whole number of sequences of length {seq}")
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for h in range(Hl):
        for b0 in range(0, T, seq):
            sl = slice(b0, b0 + seq)
            dQ[h, sl], dK[h, sl], dV[h, sl] = attention_head_bwd(Q[h, sl], K[h, sl], V[h, sl], dO3[h, sl], causal,
                                                                 None if O3 is None else O3[h, sl])
    return np.concatenate([merge_heads(dQ), merge_heads(dK), merge_heads(dV)], axis=1)
