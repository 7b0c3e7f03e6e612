"""fp64 CPU oracle for the sequence-parallel edge operations of a rank's block:
LayerNorm, and bias + dropout + residual add, each forward and backward, on
the rank's share of the tokens.

TEST INFRASTRUCTURE ONLY. This module is imported by the test suite, by the
package smoke check and by the benchmark's CPU-baseline leg. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
it imports nothing from the product path.

Sources:

* [TUT] "Megatron-LM：NVIDIA 的大规模并行训练方案", section "序列并行
  (Sequence Parallelism)": on top of tensor parallelism, LayerNorm and Dropout
  are split along the sequence dimension (each rank normalises / drops out only
  its share of the tokens), which removes the duplicated work and activation
  memory of those steps.
* [INTRO] "课程导入", section 1.4.2 (table of the four strategies): sequence
  parallelism cuts the sequence-length dimension and communicates at the
  LayerNorm / Dropout steps.
* [TUT] "融合优化技术": small elementwise steps are fused into one kernel to
  cut memory round-trips (the bias + dropout + residual add below is one such
  fusion).
* Counter-based random numbers: Philox4x32-10 as published by Salmon, Moraes,
  Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a
  10-round bijection of a 128-bit counter under a 64-bit key.

Readings taken where the pages are silent:

* LayerNorm over the hidden dimension with learned gain and bias:
  y = (x - mean) / sqrt(var + eps) * gamma + beta, var the biased variance;
  the mean and 1/sqrt(var + eps) of each row are the forward's saved outputs.
* Inverted dropout on the row-parallel output plus its bias, then the residual:
  out = residual + mask * (y + b) / (1 - p), each element kept when its
  Philox word is below floor((1 - p) 2^32).  Element e of a [rows x h] tensor
  (row-major) with stream offset o uses word (o + e) mod 4 of the Philox block
  with counter ((o + e) div 4, 0) (low 64 bits; the upper 64 bits zero) under
  key (seed low 32 bits, seed high 32 bits).  The backward regenerates the same
  mask from (seed, offset).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "PHILOX_M0", "PHILOX_M1", "PHILOX_W0", "PHILOX_W1",
    "philox4x32_10",
    "dropout_keep_threshold",
    "dropout_mask",
    "layernorm_fwd",
    "layernorm_bwd",
    "bias_dropout_add_fwd",
    "bias_dropout_add_bwd",
]

# The published round multipliers and Weyl key increments of Philox4x32.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds.  counter: uint array [..., 4]; key: [..., 2]
    (broadcast).  Returns uint32 array [..., 4].

    One round maps (c0, c1, c2, c3) under key (k0, k1) to
      (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
    the key is bumped by (W0, W1) (mod 2^32) between rounds."""
    c = np.array(counter, dtype=np.uint64) & _MASK32
    k = np.array(key, dtype=np.uint64) & _MASK32
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = k[..., 0] + np.zeros_like(c0), k[..., 1] + np.zeros_like(c0)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = np.uint64(PHILOX_M0) * c0      # < 2^64: exact in uint64
        p1 = np.uint64(PHILOX_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def dropout_keep_threshold(p: float) -> int:
    """An element is kept when its 32-bit word is below this (2^32 for p = 0)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor((1.0 - float(p)) * 4294967296.0))


def dropout_mask(rows: int, h: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean keep-mask [rows x h] of the reading in the module docstring."""
    n = rows * h
    e = np.arange(n, dtype=np.uint64) + np.uint64(offset)
    blk = e >> np.uint64(2)
    ctr = np.stack([blk & _MASK32, blk >> np.uint64(32), np.zeros_like(blk), np.zeros_like(blk)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    words = philox4x32_10(ctr, key)[np.arange(n), (e & np.uint64(3)).astype(np.int64)]
    return (words.astype(np.uint64) < np.uint64(dropout_keep_threshold(p))).reshape(rows, h)


def layernorm_fwd(X, gamma, beta=None, eps: float = 1e-5):
    """Per row of X [rows x h]: (y [rows x h], mean [rows], rstd [rows])."""
    X, g = _f64(X), _f64(gamma)
    mean = X.mean(axis=1)
    var = ((X - mean[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (X - mean[:, None]) * rstd[:, None]
    Y = xhat * g[None, :]
    if beta is not None:
        Y = Y + _f64(beta)[None, :]
    return Y, mean, rstd


def layernorm_bwd(X, gamma, dY, eps: float = 1e-5):
    """Gradients of sum(dY * y): (dX, dgamma, dbeta).  With xhat the normalised
    row and g = dY * gamma:
      dX = rstd * (g - mean_h(g) - xhat * mean_h(g * xhat)),
      dgamma = sum_rows dY * xhat,  dbeta = sum_rows dY."""
    X, g, dY = _f64(X), _f64(gamma), _f64(dY)
    _, mean, rstd = layernorm_fwd(X, g, None, eps)
    xhat = (X - mean[:, None]) * rstd[:, None]
    gy = dY * g[None, :]
    dX = rstd[:, None] * (gy - gy.mean(axis=1, keepdims=True) - xhat * (gy * xhat).mean(axis=1, keepdims=True))
    return dX, (dY * xhat).sum(axis=0), dY.sum(axis=0)


def bias_dropout_add_fwd(Y, b, residual, p: float, seed: int, offset: int):
    """out = residual + mask * (Y + b) / (1 - p); returns (out, mask)."""
    Y, R = _f64(Y), _f64(residual)
    rows, h = Y.shape
    m = dropout_mask(rows, h, p, seed, offset)
    z = Y + (_f64(b)[None, :] if b is not None else 0.0)
    return R + np.where(m, z / (1.0 - p), 0.0), m


def bias_dropout_add_bwd(dOut, p: float, seed: int, offset: int):
    """Gradients of sum(dOut * out): (dY, db, dresidual) with
    dY = mask * dOut / (1 - p), db = sum_rows dY, dresidual = dOut."""
    dOut = _f64(dOut)
    rows, h = dOut.shape
    m = dropout_mask(rows, h, p, seed, offset)
    dY = np.where(m, dOut / (1.0 - p), 0.0)
    return dY, dY.sum(axis=0), dOut
