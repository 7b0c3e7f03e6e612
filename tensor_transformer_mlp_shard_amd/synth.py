"""Seeded synthetic inputs and the workload table.

This module only draws random tensors and describes shapes. It holds none of the
method's arithmetic (no products, no activation, no reduction), so that both the
fp64 oracle's tests and the HIP path can take their inputs from it.

Every tensor is drawn on the host with a seeded ``torch.Generator`` as float32
``randn * sigma`` and then rounded to nearest-even to the storage dtype (bf16, or
kept fp32 for the fp32 workload).  Draw order is fixed per workload kind and
given in each generator below.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "seeded", "randn", "mlp_inputs", "attn_inputs", "core_attn_inputs",
           "sp_edge_inputs", "device_randn", "inputs_for"]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "mlp", "attn" (attention linears), "core_attn" or "sp_edge"
    T: int               # tokens (micro-batch x sequence, flattened)
    h: int               # hidden size
    F: int               # full FFN width (mlp) or full QKV width (attn)
    tp: int              # tensor-parallel degree
    dtype: str           # "bf16", "fp16" or "fp32"
    sigma_w: float       # weight / bias std
    seed: int
    full: bool           # draw unsharded weights (then slice) or the rank's shard only
    note: str = field(default="", compare=False)
    seq: int = 0         # core_attn: sequence length (T = micro-batch x seq)
    heads: int = 0       # core_attn: attention heads of the whole layer

    @property
    def f(self) -> int:
        return self.F // self.tp

    @property
    def heads_local(self) -> int:
        return self.heads // self.tp

    @property
    def head_dim(self) -> int:
        return self.h // self.heads


# Sizes follow the pages' workloads: the GPT launch example of the tutorial
# (24 layers, hidden 1024, 16 heads, sequence 1024, micro-batch 4, TP=2), the
# 1.3B single-GPU case of the course introduction (hidden 2048, sequence 1024,
# micro-batch 4) and the 175B tensor-parallel case (hidden 12288, QKV
# 12288 x 36864 in 8 shards of 12288 x 4608).  FFN width = 4 x hidden.
WORKLOADS = {
    "tiny_tp2_fp32": Workload("tiny_tp2_fp32", "mlp", 128, 256, 1024, 2, "fp32", 0.02, 1235, True,
                              "X[128x256], A_i[256x512], B_i[512x256]; unsharded A[256x1024] too"),
    "gpt_h1024_tp2": Workload("gpt_h1024_tp2", "mlp", 4096, 1024, 4096, 2, "bf16", 0.02, 1236, True,
                              "GPT 24-layer h=1024, seq 1024 x micro-batch 4, TP=2 rank MLP shard"),
    "gpt_1p3b_tp1": Workload("gpt_1p3b_tp1", "mlp", 4096, 2048, 8192, 1, "bf16", 0.02, 1237, True,
                             "1.3B GPT h=2048 ffn=8192, seq 1024 x micro-batch 4, TP=1 (whole MLP)"),
    "gpt175b_mlp_tp8": Workload("gpt175b_mlp_tp8", "mlp", 2048, 12288, 49152, 8, "bf16", 0.006, 1238, False,
                                "175B MLP shard at TP=8: X[2048x12288], A_i[12288x6144], B_i[6144x12288]"),
    "gpt175b_attn_tp8": Workload("gpt175b_attn_tp8", "attn", 8192, 12288, 36864, 8, "bf16", 0.006, 1239, False,
                                 "175B attention linears at TP=8: QKV 12288->4608 column shard, "
                                 "out-proj 1536->12288 row shard"),
    # Core attention on a rank's local heads.  Head counts: 16 for the tutorial's
    # GPT (head dim 64); 96 for the 175B case (head dim 128, so the 4608-wide
    # QKV shard holds 12 heads).  The 175B token count is 4 sequences of 2048.
    # QKV activations are drawn N(0, 1), which puts the scaled scores at unit
    # spread.
    "gpt_h1024_core_attn_tp2": Workload("gpt_h1024_core_attn_tp2", "core_attn", 4096, 1024, 3072, 2, "bf16", 1.0,
                                        1240, False, "GPT h=1024 TP=2: 8 local heads of 64, 4 x 1024 tokens",
                                        seq=1024, heads=16),
    "gpt175b_core_attn_tp8": Workload("gpt175b_core_attn_tp8", "core_attn", 8192, 12288, 36864, 8, "bf16", 1.0,
                                      1241, False, "175B TP=8: 12 local heads of 128, 4 x 2048 tokens",
                                      seq=2048, heads=96),
    # Sequence-parallel edge steps on the rank's share of the tokens: T here is
    # that share (all tokens / tp), h the hidden size.
    "gpt_h1024_sp_edge_tp2": Workload("gpt_h1024_sp_edge_tp2", "sp_edge", 2048, 1024, 0, 2, "bf16", 0.02, 1242,
                                      False, "GPT h=1024 TP=2: 4096 tokens / 2 rows of 1024"),
    "gpt175b_sp_edge_tp8": Workload("gpt175b_sp_edge_tp8", "sp_edge", 1024, 12288, 0, 8, "bf16", 0.006, 1243,
                                    False, "175B TP=8: 8192 tokens / 8 rows of 12288"),
}

_TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32, "fp16": torch.float16}


def seeded(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(gen: torch.Generator, shape, sigma: float, dtype: str) -> torch.Tensor:
    """float32 N(0, sigma^2) draw, rounded to ``dtype`` (round-to-nearest-even)."""
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(_TORCH_DTYPE[dtype]).contiguous()


def device_randn(shape, sigma: float, dtype: str, seed: int, device) -> torch.Tensor:
    """Seeded N(0, sigma^2) draw made on the device (for inputs too large to
    draw on the host), rounded to ``dtype``.  The same seed and shape give the
    same bits on the same device type."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(_TORCH_DTYPE[dtype])


def mlp_inputs(T: int, h: int, F: int, tp: int, dtype: str, sigma_w: float, seed: int,
               full: bool = True, sigma_x: float = 1.0, sigma_dy: float = 1.0) -> dict:
    """Inputs of one MLP shard.  Draw order: X, A, b1, B, b2, dY.

    With ``full`` the unsharded A[h x F], b1[F], B[F x h] are drawn (callers take
    rank shards by slicing); otherwise A, b1, B are already the rank's shard of
    width f = F / tp.  b2[h] is the row-parallel output bias.
    """
    if F % tp:
        raise ValueError("F must be divisible by tp")
    width = F if full else F // tp
    g = seeded(seed)
    out = {}
    out["X"] = randn(g, (T, h), sigma_x, dtype)
    out["A"] = randn(g, (h, width), sigma_w, dtype)
    out["b1"] = randn(g, (width,), sigma_w, dtype)
    out["B"] = randn(g, (width, h), sigma_w, dtype)
    out["b2"] = randn(g, (h,), sigma_w, dtype)
    out["dY"] = randn(g, (T, h), sigma_dy, dtype)
    out["full"] = full
    return out


def attn_inputs(T: int, h: int, qkv_width: int, tp: int, dtype: str, sigma_w: float, seed: int) -> dict:
    """Inputs of the two attention-linear shards (rank shards drawn directly).

    Draw order: X[T x h], W_qkv[h x qkv/tp], b_qkv[qkv/tp], O[T x h/tp],
    W_o[h/tp x h], b_o[h], dQKV[T x qkv/tp], dY[T x h].
    """
    if qkv_width % tp or h % tp:
        raise ValueError("widths must be divisible by tp")
    g = seeded(seed)
    q = qkv_width // tp
    k = h // tp
    out = {}
    out["X"] = randn(g, (T, h), 1.0, dtype)
    out["W_qkv"] = randn(g, (h, q), sigma_w, dtype)
    out["b_qkv"] = randn(g, (q,), sigma_w, dtype)
    out["O"] = randn(g, (T, k), 1.0, dtype)
    out["W_o"] = randn(g, (k, h), sigma_w, dtype)
    out["b_o"] = randn(g, (h,), sigma_w, dtype)
    out["dQKV"] = randn(g, (T, q), 1.0, dtype)
    out["dY"] = randn(g, (T, h), 1.0, dtype)
    return out


def core_attn_inputs(T: int, heads_local: int, head_dim: int, dtype: str, sigma: float, seed: int) -> dict:
    """Inputs of core attention on one rank's heads.

    Draw order: QKV[T x 3*Hl*d] (columns [Q | K | V], head-major in each),
    dO[T x Hl*d].  QKV entries are N(0, sigma^2), dO entries N(0, 1).
    """
    g = seeded(seed)
    w = heads_local * head_dim
    return {"QKV": randn(g, (T, 3 * w), sigma, dtype), "dO": randn(g, (T, w), 1.0, dtype)}


def sp_edge_inputs(rows: int, h: int, dtype: str, sigma_w: float, seed: int) -> dict:
    """Inputs of the sequence-parallel edge steps on a rank's rows.

    Draw order: X[rows x h] (LayerNorm input), gamma[h] = 1 + N(0, 0.1^2),
    beta[h] ~ N(0, 0.1^2), dY_ln[rows x h], Y[rows x h] (row-parallel output),
    b[h] ~ N(0, sigma_w^2), residual[rows x h], dOut[rows x h]; the rest N(0, 1).
    """
    g = seeded(seed)
    out = {"X": randn(g, (rows, h), 1.0, dtype)}
    gam = torch.randn(h, generator=g, dtype=torch.float32) * 0.1 + 1.0
    out["gamma"] = gam.to(_TORCH_DTYPE[dtype]).contiguous()
    out["beta"] = randn(g, (h,), 0.1, dtype)
    out["dY_ln"] = randn(g, (rows, h), 1.0, dtype)
    out["Y"] = randn(g, (rows, h), 1.0, dtype)
    out["b"] = randn(g, (h,), sigma_w, dtype)
    out["residual"] = randn(g, (rows, h), 1.0, dtype)
    out["dOut"] = randn(g, (rows, h), 1.0, dtype)
    return out


def inputs_for(w: Workload) -> dict:
    if w.kind == "sp_edge":
        return sp_edge_inputs(w.T, w.h, w.dtype, w.sigma_w, w.seed)
    if w.kind == "core_attn":
        return core_attn_inputs(w.T, w.heads_local, w.head_dim, w.dtype, w.sigma_w, w.seed)
    if w.kind == "mlp":
        return mlp_inputs(w.T, w.h, w.F, w.tp, w.dtype, w.sigma_w, w.seed, full=w.full)
    return attn_inputs(w.T, w.h, w.F, w.tp, w.dtype, w.sigma_w, w.seed)
