"""fp64 CPU oracle for one rank's share of a tensor-parallel Transformer block.

TEST INFRASTRUCTURE ONLY. This module is imported by the test suite, by the
package smoke check and by the benchmark's CPU-baseline leg. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
it imports nothing from the product path.

Sources (the web pages this method is described on):

* [TUT]  "Megatron-LM：NVIDIA 的大规模并行训练方案" (freeguideonline Megatron-LM
  tutorial), section "Megatron-LM 核心架构 / 张量并行原理" (tensor-parallel
  principle): the linear layer Y = XA; column-parallel split A = [A_1, A_2],
  Y_i = X A_i; row-parallel split (A by rows, X by columns, local products summed
  by AllReduce); in a Transformer the QKV projection and the MLP's first layer
  are column-parallel, the attention output projection and the MLP's second
  layer are row-parallel.  Section "融合优化技术" (fused optimisations): bias and
  GeLU are fused into one kernel to cut memory round-trips.
* [BASICS] "分布式训练基础：数据并行、模型并行、流水线并行的基本概念与区别",
  section 2.2 "模型并行 —— 张量并行", "核心原理": the same column split
  Y = XW, W = [W1, W2], each device computes X W_i; the row split W = [W1; W2],
  X = [X1, X2], each device computes X_i W_i and an AllReduce sums them; the
  same Transformer placement.  "案例拆解：175B 的张量并行": the 175B QKV matrix
  12288 x 36864 cut into 8 shards of 12288 x 4608.

Readings taken where the pages are silent:

* GeLU is the exact one, GeLU(z) = z * Phi(z) with Phi the standard normal CDF
  (the pages only say "GeLU").
* Weights are [in x out] row-major, as in Y = XA; rank i owns the contiguous
  column block i (column-parallel) or row block i (row-parallel).
* The row-parallel partial Y_i carries no output bias; the bias is added once
  after the sum, so its gradient sum_t dY is computed once.
* The pages give no backward formulas; the backward here is the chain rule of
  the forward, and is pinned by finite differences in the tests.

Everything is computed in float64 from the given inputs, with no intermediate
rounding.  Matrix products use numpy's float64 matmul as a library primitive;
there is no blocking, fusion or reordering beyond the formulas written below.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "std_normal_cdf",
    "std_normal_pdf",
    "gelu",
    "gelu_grad",
    "column_shard",
    "row_shard",
    "column_linear_fwd",
    "row_linear_fwd",
    "mlp_shard_fwd",
    "mlp_shard_bwd",
    "linear_bwd",
    "bias_grad",
    "bias_gelu",
    "rel_fro",
]

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Activation ([TUT] "融合优化技术": bias + GeLU; exact-erf reading)
# --------------------------------------------------------------------------
def std_normal_cdf(z):
    """Phi(z) = (1 + erf(z / sqrt 2)) / 2."""
    z = _f64(z)
    return 0.5 * (1.0 + _erf(z / _SQRT2))


def std_normal_pdf(z):
    """phi(z) = exp(-z^2 / 2) / sqrt(2 pi)."""
    z = _f64(z)
    return np.exp(-0.5 * z * z) * _INV_SQRT_2PI


def gelu(z):
    """GeLU(z) = z * Phi(z) (exact, erf-based)."""
    z = _f64(z)
    return z * std_normal_cdf(z)


def gelu_grad(z):
    """d GeLU / dz = Phi(z) + z * phi(z)  (product rule on z * Phi(z))."""
    z = _f64(z)
    return std_normal_cdf(z) + z * std_normal_pdf(z)


# --------------------------------------------------------------------------
# Sharding ([TUT] "张量并行原理"; [BASICS] 2.2 "核心原理")
# --------------------------------------------------------------------------
def column_shard(W, tp_size: int, rank: int) -> np.ndarray:
    """Column-parallel shard: W = [W_1, ..., W_p] split by columns; rank i
    keeps the contiguous block of out/p columns number i."""
    W = np.asarray(W)
    n = W.shape[-1]
    if n % tp_size:
        raise ValueError("out-features not divisible by the TP degree")
    w = n // tp_size
    return W[..., rank * w:(rank + 1) * w]


def row_shard(W, tp_size: int, rank: int) -> np.ndarray:
    """Row-parallel shard: W = [W_1; ...; W_p] split by rows; rank i keeps the
    contiguous block of in/p rows number i (and the matching column block of X,
    which is column_shard(X, p, i))."""
    W = np.asarray(W)
    k = W.shape[0]
    if k % tp_size:
        raise ValueError("in-features not divisible by the TP degree")
    w = k // tp_size
    return W[rank * w:(rank + 1) * w]


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------
def column_linear_fwd(X, W_i, b_i=None, act: str = "none"):
    """Column-parallel linear on rank i: Z_i = X W_i (+ b_i), Y_i = act(Z_i).

    X is the replicated input [T x K]; W_i is the rank's column block [K x N/p].
    Returns (Z_i, Y_i); with act == "none" they are the same array.
    [TUT] "张量并行原理" (Y_i = X A_i); [BASICS] 2.2 "核心原理".
    """
    X = _f64(X)
    W_i = _f64(W_i)
    Z = X @ W_i
    if b_i is not None:
        Z = Z + _f64(b_i)[None, :]
    if act == "none":
        return Z, Z
    if act == "gelu":
        return Z, gelu(Z)
    raise ValueError(f"unknown activation {act!r}")


def row_linear_fwd(X_i, W_i, b=None):
    """Row-parallel linear on rank i: the partial Y_i = X_i W_i, where X_i is the
    rank's column block of the input [T x K/p] and W_i the row block [K/p x N].
    The sum over ranks of Y_i is the full product.  The output bias b, when
    given, is added here (the caller passes it on exactly one rank).
    [TUT] "张量并行原理" (row split + AllReduce sum); [BASICS] 2.2 "核心原理".
    """
    Y = _f64(X_i) @ _f64(W_i)
    if b is not None:
        Y = Y + _f64(b)[None, :]
    return Y


def mlp_shard_fwd(X, A_i, b1_i, B_i):
    """One rank's share of the tensor-parallel MLP.

    First layer column-parallel, second layer row-parallel ([TUT] "张量并行原理",
    last paragraph; [BASICS] 2.2), with the bias + GeLU between them ([TUT]
    "融合优化技术"):
        Z_i = X A_i + b1_i          [T x F/p]
        H_i = GeLU(Z_i)             [T x F/p]
        Y_i = H_i B_i               [T x h], partial: the row-parallel sum over
                                    ranks (and the output bias) come later.
    Returns (Z_i, H_i, Y_i).
    """
    Z, H = column_linear_fwd(X, A_i, b1_i, act="gelu")
    Y = H @ _f64(B_i)
    return Z, H, Y


# --------------------------------------------------------------------------
# Backward (chain rule of the forward above)
# --------------------------------------------------------------------------
def mlp_shard_bwd(X, A_i, b1_i, B_i, dY):
    """Gradients of one rank's MLP share, given dY = dL/dY (the gradient of the
    summed output, replicated on every rank).

        Z_i, H_i  recomputed exactly from the inputs
        dB_i  = H_i^T dY
        dH_i  = dY B_i^T
        dZ_i  = dH_i * GeLU'(Z_i)
        db1_i = sum_t dZ_i[t, :]
        dA_i  = X^T dZ_i
        dX_i  = dZ_i A_i^T   (this rank's partial of dX; the column-parallel
                              backward sums it over ranks)
    Returns dict(dX, dA, db1, dB, dZ, Z, H).
    """
    X = _f64(X)
    A_i = _f64(A_i)
    B_i = _f64(B_i)
    dY = _f64(dY)
    Z, H, _ = mlp_shard_fwd(X, A_i, b1_i, B_i)
    dB = H.T @ dY
    dH = dY @ B_i.T
    dZ = dH * gelu_grad(Z)
    db1 = dZ.sum(axis=0)
    dA = X.T @ dZ
    dX = dZ @ A_i.T
    return {"dX": dX, "dA": dA, "db1": db1, "dB": dB, "dZ": dZ, "Z": Z, "H": H}


def linear_bwd(X, W, dY):
    """Gradients of Y = X W (+ b) for either shard kind: with X [T x K],
    W [K x N], dY [T x N]:
        dX = dY W^T,  dW = X^T dY,  db = sum_t dY[t, :].
    For a column shard, X is the replicated input and dX is this rank's partial;
    for a row shard, X is the rank's input block and dX is its exact gradient.
    Returns dict(dX, dW, db).
    """
    X = _f64(X)
    W = _f64(W)
    dY = _f64(dY)
    return {"dX": dY @ W.T, "dW": X.T @ dY, "db": dY.sum(axis=0)}


def bias_grad(dY):
    """sum over tokens of dY: the gradient of a bias added to every row."""
    return _f64(dY).sum(axis=0)


def bias_gelu(Z, b):
    """The unfused elementwise step: H = GeLU(Z + b) (b broadcast over rows)."""
    return gelu(_f64(Z) + _f64(b)[None, :])


# --------------------------------------------------------------------------
# Error metric
# --------------------------------------------------------------------------
def rel_fro(got, ref) -> float:
    """||got - ref||_F / ||ref||_F, computed in float64."""
    got = _f64(got)
    ref = _f64(ref)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(got - ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den
