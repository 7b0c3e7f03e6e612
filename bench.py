"""Throughput of one rank's tensor-parallel Transformer-layer shard, fwd + bwd, bf16.

One step runs every operation of the shard once, through the C ABI, on
synthetic inputs already resident in HBM:
  * the 175B-shaped MLP shard at TP=8 (T=2048 tokens, h=12288, f=6144):
    forward (X A_i + b1 -> GeLU -> H B_i) and backward (dZ with GeLU', dB, dA,
    dX, db1, db2);
  * the 175B-shaped attention linears at TP=8 (T=8192 tokens): the QKV column
    shard (12288 -> 4608, with bias) and the output-projection row shard
    (1536 -> 12288), each forward and backward (dX, dW, db).
The metric is algorithmic matrix FLOP per step (2 M N K per product) divided by
the step time, in TFLOP/s, and its fraction of the MI355X dense bf16 matrix
peak (2.5 PFLOP/s).

Prints one JSON line.  Extra fields: per-part times, a roofline entry for the
kernel with the most time in the step (timed with HIP events around its
launches by the library's trace), the register-only matrix-core probe, the
fp64 CPU oracle timed on a bounded sample of the same workload, and, outside
the step, the same step in fp16, core attention on the rank's local heads (175B
shape: 4 sequences of 2048 tokens, 12 heads of 128, causal) forward and
backward, the selective
recompute forms of the MLP backward, the sequence-parallel edge steps
(LayerNorm, bias + dropout + residual) in GB/s, and, for context, the step's
12 matrix products through the vendor library (torch.mm -> hipBLASLt).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0
METRIC = "TFLOP/s per TP shard fwd+bwd (bf16) + % of MI355X bf16 MFMA peak"


def _flops_mlp(T, h, f):
    return 2.0 * T * h * f * 2 * 3      # 2 forward + 4 backward products, each 2 T h f


def _flops_attn(T, h, q, k):
    qkv = 2.0 * T * h * q
    proj = 2.0 * T * k * h
    return 3 * qkv + 3 * proj


class Shard:
    """Device-resident inputs, outputs and workspaces of the two parts."""

    def __init__(self, device, dtype: str = "bf16"):
        import dataclasses

        import torch

        import tensor_transformer_mlp_shard_amd as tps
        from tensor_transformer_mlp_shard_amd import _native, synth

        self.tps = tps
        self.torch = torch
        wm = dataclasses.replace(synth.WORKLOADS["gpt175b_mlp_tp8"], dtype=dtype)
        wa = dataclasses.replace(synth.WORKLOADS["gpt175b_attn_tp8"], dtype=dtype)
        self.wm, self.wa = wm, wa
        m = synth.inputs_for(wm)
        a = synth.inputs_for(wa)
        self.host_mlp, self.host_attn = m, a
        d = lambda t: t.to(device)  # noqa: E731
        self.X, self.A, self.b1, self.B, self.dY = (d(m[k]) for k in ("X", "A", "b1", "B", "dY"))
        self.Xa, self.Wq, self.bq, self.O, self.Wo, self.dQ, self.dYa = (
            d(a[k]) for k in ("X", "W_qkv", "b_qkv", "O", "W_o", "dQKV", "dY"))
        T, h, f, p = wm.T, wm.h, wm.f, wm.tp
        bf, fp = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype], torch.float32
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)  # noqa: E731
        self.fwd_out = {"Z": e((T, f), bf), "H": e((T, f), bf), "Y": e((T, h), bf)}
        self.bwd_out = {"dX": e((T, h), bf), "dA": e((h, f), fp), "dB": e((f, h), fp), "db1": e((f,), fp),
                        "db2": e((h,), fp)}
        self.ws_mlp = e((tps.workspace_size(_native.TP_OP_MLP_SHARD_BWD, T, h, wm.F, p, bf),), torch.uint8)
        Ta, ha, q, k = wa.T, wa.h, wa.F // wa.tp, wa.h // wa.tp
        self.q_out = {"dX": e((Ta, ha), bf), "dW": e((ha, q), fp), "db": e((q,), fp)}
        self.o_out = {"dX": e((Ta, k), bf), "dW": e((k, ha), fp), "db": e((ha,), fp)}
        self.ws_q = e((tps.workspace_size(_native.TP_OP_COLUMN_LINEAR_BWD, Ta, ha, wa.F, wa.tp, bf),), torch.uint8)
        self.ws_o = e((tps.workspace_size(_native.TP_OP_ROW_LINEAR_BWD, Ta, ha, ha, wa.tp, bf),), torch.uint8)
        self.flops_mlp = _flops_mlp(T, h, f)
        self.flops_attn = _flops_attn(Ta, ha, q, k)

    def mlp_step(self):
        tps = self.tps
        o = self.fwd_out
        tps.mlp_shard_fwd(self.X, self.A, self.b1, self.B, tp_size=self.wm.tp, out=o)
        tps.mlp_shard_bwd(self.X, self.A, self.B, o["Z"], o["H"], self.dY, tp_size=self.wm.tp, want_db2=True,
                          out=self.bwd_out, workspace=self.ws_mlp)

    def attn_step(self):
        tps = self.tps
        p = self.wa.tp
        tps.column_linear(self.Xa, self.Wq, self.bq, tp_size=p)
        tps.column_linear_bwd(self.Xa, self.Wq, self.dQ, tp_size=p, out=self.q_out, workspace=self.ws_q)
        tps.row_linear(self.O, self.Wo, None, tp_size=p)
        tps.row_linear_bwd(self.O, self.Wo, self.dYa, tp_size=p, out=self.o_out, workspace=self.ws_o)

    def step(self):
        self.mlp_step()
        self.attn_step()


class MLPConfig:
    """One rank's MLP shard of a workload in the table (rank 0's contiguous
    column block of A and b1 and row block of B when the unsharded weights are
    drawn), device-resident, with preallocated outputs and workspace; one step
    is the forward and the backward (dX, dA, db1, dB, db2)."""

    def __init__(self, device, name: str):
        import torch

        import tensor_transformer_mlp_shard_amd as tps
        from tensor_transformer_mlp_shard_amd import _native, synth

        self.tps = tps
        w = synth.WORKLOADS[name]
        self.w = w
        d = synth.inputs_for(w)
        f = w.f
        if w.full:   # rank 0's shard of the unsharded weights
            d["A"], d["b1"], d["B"] = d["A"][:, :f].contiguous(), d["b1"][:f].contiguous(), d["B"][:f].contiguous()
        self.X, self.A, self.b1, self.B, self.dY = (d[k].to(device) for k in ("X", "A", "b1", "B", "dY"))
        dt = self.X.dtype
        e = lambda shape, t: torch.empty(shape, dtype=t, device=device)  # noqa: E731
        T, h = w.T, w.h
        self.fwd_out = {"Z": e((T, f), dt), "H": e((T, f), dt), "Y": e((T, h), dt)}
        fp = torch.float32
        self.bwd_out = {"dX": e((T, h), dt), "dA": e((h, f), fp), "dB": e((f, h), fp), "db1": e((f,), fp),
                        "db2": e((h,), fp)}
        self.ws = e((tps.workspace_size(_native.TP_OP_MLP_SHARD_BWD, T, h, w.F, w.tp, dt),), torch.uint8)
        self.flops = _flops_mlp(T, h, f)

    def step(self):
        o = self.fwd_out
        self.tps.mlp_shard_fwd(self.X, self.A, self.b1, self.B, tp_size=self.w.tp, out=o)
        self.tps.mlp_shard_bwd(self.X, self.A, self.B, o["Z"], o["H"], self.dY, tp_size=self.w.tp, want_db2=True,
                               out=self.bwd_out, workspace=self.ws)


def _kernel_breakdown(tps, torch, fn, steps):
    """Per-kernel HIP-event times of `steps` calls of fn (the library's trace)."""
    tps.trace_start(4096)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return [{"name": k["name"], "launches_per_step": k["launches"] // steps,
             "us_per_step": round(1e3 * k["total_ms"] / steps, 2),
             "tflops": round(k["flops"] / (k["total_ms"] * 1e-3) / 1e12, 1) if k["flops"] else None}
            for k in tps.trace_stop()]


def measure_configs(torch, device, shard, steps, warmup):
    """Forward + backward of every workload in the table, each on its own:
    the tiny fp32 check-path shard, the GPT h=1024 TP=2 and 1.3B TP=1 MLP
    shards, and the two 175B TP=8 parts of the step (MLP shard, attention
    linears).  TFLOP/s and % of the bf16 peak from the median step."""
    out = {}
    for key, name in (("tiny_tp2_fp32", "tiny_tp2_fp32"), ("gpt_h1024_tp2_mlp", "gpt_h1024_tp2"),
                      ("gpt_1p3b_tp1_mlp", "gpt_1p3b_tp1")):
        c = MLPConfig(device, name)
        st = time_stats(torch, c.step, steps, warmup)
        w = c.w
        out[key] = {"workload": f"{w.note}: X[{w.T}x{w.h}], A_i[{w.h}x{w.f}], B_i[{w.f}x{w.h}], fwd+bwd",
                    "dtype": w.dtype, "flop": c.flops, **_rates(c.flops, st)}
        if w.dtype == "fp32":
            out[key]["note"] = "fp32 check path (FMA kernel, not the matrix cores): latency-bound, parity only"
        else:
            out[key]["kernels"] = _kernel_breakdown(c.tps, torch, c.step, steps)
        del c
    st = time_stats(torch, shard.mlp_step, steps, warmup)
    out["gpt175b_mlp_tp8"] = {"workload": "175B MLP shard at TP=8: X[2048x12288], A_i[12288x6144], "
                                          "B_i[6144x12288], fwd+bwd", "dtype": "bf16", "flop": shard.flops_mlp,
                              **_rates(shard.flops_mlp, st)}
    st = time_stats(torch, shard.attn_step, steps, warmup)
    out["gpt175b_attn_tp8"] = {"workload": "175B attention linears at TP=8, T=8192: QKV 12288->4608 (bias), "
                                           "out-proj 1536->12288, fwd+bwd", "dtype": "bf16",
                               "flop": shard.flops_attn, **_rates(shard.flops_attn, st)}
    return out


class CoreAttention:
    """Core attention on the rank's local heads, 175B shape at TP=8: 4 sequences
    of 2048 tokens, 12 local heads of 128, causal; forward and backward."""

    def __init__(self, device):
        import torch

        import tensor_transformer_mlp_shard_amd as tps
        from tensor_transformer_mlp_shard_amd import _native, synth

        self.tps = tps
        w = synth.WORKLOADS["gpt175b_core_attn_tp8"]
        self.w = w
        x = synth.inputs_for(w)
        self.qkv, self.dO = x["QKV"].to(device), x["dO"].to(device)
        W = w.heads_local * w.head_dim
        self.O = torch.empty((w.T, W), dtype=torch.bfloat16, device=device)
        self.dqkv = torch.empty((w.T, 3 * W), dtype=torch.bfloat16, device=device)
        self.ws = torch.empty((tps.workspace_size(_native.TP_OP_ATTENTION_BWD, w.T, w.heads, w.head_dim, w.tp,
                                                  torch.bfloat16),), dtype=torch.uint8, device=device)
        self.kw = dict(seq=w.seq, heads=w.heads, head_dim=w.head_dim, tp_size=w.tp, causal=True)
        pairs = w.seq * (w.seq + 1) / 2 * (w.T // w.seq) * w.heads_local
        self.flops_fwd = 4.0 * w.head_dim * pairs            # Q K^T and P V
        self.flops_bwd = 2.5 * self.flops_fwd                # dV, dP, dQ, dK (+ S recomputed: not counted)
        self.lse = None
        self.fwd()

    def fwd(self):
        _, self.lse = self.tps.attention_fwd(self.qkv, out=self.O, **self.kw)

    def bwd(self):
        self.tps.attention_bwd(self.qkv, self.O, self.lse, self.dO, out=self.dqkv, workspace=self.ws, **self.kw)

    def step(self):
        self.fwd()
        self.bwd()


def measure_vendor_gemms(torch, shard, steps, warmup):
    """The step's 12 matrix products through torch.mm (hipBLASLt on ROCm), bf16
    in and out, on the same resident tensors: context for the hand-written
    kernels, not a measurement of this library (no epilogues, no bias
    gradients, bf16 instead of fp32 weight-gradient outputs)."""
    X, A, B, dY = shard.X, shard.A, shard.B, shard.dY
    H, Z = shard.fwd_out["H"], shard.fwd_out["Z"]
    Xa, Wq, dQ, O, Wo, dYa = shard.Xa, shard.Wq, shard.dQ, shard.O, shard.Wo, shard.dYa
    prods = [(X, A), (H, B), (dY, B.t()), (H.t(), dY), (X.t(), Z), (Z, A.t()),
             (Xa, Wq), (dQ, Wq.t()), (Xa.t(), dQ), (O, Wo), (dYa, Wo.t()), (O.t(), dYa)]
    outs = [torch.empty((a.shape[0], b.shape[1]), dtype=a.dtype, device=a.device) for a, b in prods]
    flops = sum(2.0 * a.shape[0] * a.shape[1] * b.shape[1] for a, b in prods)

    def run():
        for (a, b), c in zip(prods, outs):
            torch.mm(a, b, out=c)

    ms, _ = time_steps(torch, run, steps, warmup)
    names = ["fc1", "fc2", "mlp_dH", "mlp_dB", "mlp_dA", "mlp_dX", "qkv", "qkv_dX", "qkv_dW", "oproj", "oproj_dX",
             "oproj_dW"]
    each = []
    for name, (a, b), c in zip(names, prods, outs):
        pms, _ = time_steps(torch, lambda a=a, b=b, c=c: torch.mm(a, b, out=c), steps, 3)
        f = 2.0 * a.shape[0] * a.shape[1] * b.shape[1]
        each.append({"gemm": name, "m_n_k": [a.shape[0], b.shape[1], a.shape[1]], "ms": round(pms, 4),
                     "tflops": round(f / (pms * 1e-3) / 1e12, 1)})
    return {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "flop": flops, "per_product": each,
            "note": "the step's 12 products via torch.mm (hipBLASLt), bf16 in/out, no epilogues or bias "
                    "gradients: vendor-library context, not this library"}


def measure_core_attention(torch, device, steps, warmup):
    ca = CoreAttention(device)
    out = {"workload": "175B TP=8 core attention: 4 x 2048 tokens, 12 local heads of 128, causal, bf16",
           "flop_fwd": ca.flops_fwd, "flop_bwd": ca.flops_bwd}
    for name, fn, fl in (("fwd", ca.fwd, ca.flops_fwd), ("bwd", ca.bwd, ca.flops_bwd),
                         ("fwd_bwd", ca.step, ca.flops_fwd + ca.flops_bwd)):
        out[name] = _rates(fl, time_stats(torch, fn, steps, warmup))
    ca.tps.trace_start(4096)
    for _ in range(steps):
        ca.step()
    torch.cuda.synchronize()
    out["kernels"] = [{"name": k["name"], "launches_per_step": k["launches"] // steps,
                       "ms_per_step": round(k["total_ms"] / steps, 4),
                       "tflops": round(k["flops"] / (k["total_ms"] * 1e-3) / 1e12, 1) if k["flops"] else None,
                       "gbs": round(k["bytes"] / (k["total_ms"] * 1e-3) / 1e9, 1)}
                      for k in ca.tps.trace_stop()]
    return out


def measure_sp_edge(torch, device, steps, warmup):
    """Sequence-parallel edge steps on the 175B rank's rows (8192 tokens / 8 =
    1024 rows of 12288), HBM-bound: GB/s of algorithmic traffic per kernel."""
    import tensor_transformer_mlp_shard_amd as tps
    from tensor_transformer_mlp_shard_amd import synth

    w = synth.WORKLOADS["gpt175b_sp_edge_tp8"]
    x = {k: v.to(device) for k, v in synth.inputs_for(w).items()}
    y, mean, rstd = tps.layernorm_fwd(x["X"], x["gamma"], x["beta"])
    lnb = {"dX": torch.empty_like(x["X"]), "dgamma": torch.empty(w.h, device=device),
           "dbeta": torch.empty(w.h, device=device)}
    out = torch.empty_like(x["Y"])
    dy = torch.empty_like(x["Y"])

    def step():
        tps.layernorm_fwd(x["X"], x["gamma"], x["beta"], out=y)
        tps.layernorm_bwd(x["X"], x["gamma"], mean, rstd, x["dY_ln"], out=lnb)
        tps.bias_dropout_add_fwd(x["Y"], x["b"], x["residual"], p=0.1, seed=1, offset=0, out=out)
        tps.bias_dropout_add_bwd(x["dOut"], p=0.1, seed=1, offset=0, out=dy)

    ms, _ = time_steps(torch, step, steps, warmup)
    tps.trace_start(4096)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern = [{"name": k["name"], "launches_per_step": k["launches"] // steps,
             "us_per_step": round(1e3 * k["total_ms"] / steps, 2),
             "gbs": round(k["bytes"] / (k["total_ms"] * 1e-3) / 1e9, 1),
             "frac_hbm": round(k["bytes"] / (k["total_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
            for k in tps.trace_stop()]
    return {"workload": f"175B TP=8 sequence-parallel rows: {w.T} x {w.h}, bf16, dropout p=0.1",
            "ms_per_step": round(ms, 4), "kernels": kern}


def measure_side(torch, device, steps, warmup):
    """The HBM-bound side kernels on the 175B MLP shard's shapes: the replicated
    row-parallel bias gradient db2 = sum_t dY over dY [2048 x 12288] (column-sum
    pass + fixed-order finalize) and the unfused H = GeLU(Z + b1) over
    Z [2048 x 6144] that the fused fc1 epilogue replaces: GB/s of algorithmic
    traffic per kernel."""
    import tensor_transformer_mlp_shard_amd as tps
    from tensor_transformer_mlp_shard_amd import _native, synth

    w = synth.WORKLOADS["gpt175b_mlp_tp8"]
    f = w.F // w.tp
    g = synth.seeded(w.seed + 7)
    dY = synth.randn(g, (w.T, w.h), 1.0, "bf16").to(device)
    Z = synth.randn(g, (w.T, f), 1.0, "bf16").to(device)
    b1 = synth.randn(g, (f,), 0.02, "bf16").to(device)
    ws = torch.empty(tps.workspace_size(_native.TP_OP_BIAS_GRAD, w.T, w.h, 0, 1, torch.bfloat16), dtype=torch.uint8,
                     device=device)

    def step():
        tps.bias_grad(dY, workspace=ws)
        tps.bias_gelu(Z, b1)

    ms, _ = time_steps(torch, step, steps, warmup)
    tps.trace_start(4096)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern = [{"name": k["name"], "launches_per_step": k["launches"] // steps,
             "us_per_step": round(1e3 * k["total_ms"] / steps, 2),
             "gbs": round(k["bytes"] / (k["total_ms"] * 1e-3) / 1e9, 1),
             "frac_hbm": round(k["bytes"] / (k["total_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
            for k in tps.trace_stop()]
    return {"workload": f"db2 = sum_t dY over {w.T} x {w.h} and GeLU(Z + b1) over {w.T} x {f}, bf16",
            "ms_per_step": round(ms, 4), "kernels": kern}


def measure_recompute(torch, shard, steps, warmup, pairs=6):
    """MLP shard fwd+bwd with all activations saved against the two selective
    recompute forms: Z kept (H recomputed by an elementwise GeLU) and nothing
    kept (Z and H recomputed by the fc1 GEMM).  The three forms run in turn,
    `pairs` rounds of `steps` steps each, so that each overhead is a paired
    difference against the baseline round next to it; reported as the median
    and the range over the rounds, with the activation bytes each form keeps
    between forward and backward."""
    tps = shard.tps
    wm = shard.wm
    p = wm.tp
    o = shard.fwd_out
    ws = torch.empty((tps.workspace_size(tps._native.TP_OP_MLP_SHARD_BWD_RECOMPUTE, wm.T, wm.h, wm.F, p,
                                         torch.bfloat16),), dtype=torch.uint8, device=shard.X.device)

    def keep_z():
        tps.mlp_shard_fwd(shard.X, shard.A, shard.b1, shard.B, tp_size=p, out=o)
        tps.mlp_shard_bwd(shard.X, shard.A, shard.B, o["Z"], None, shard.dY, tp_size=p, want_db2=True,
                          out=shard.bwd_out, workspace=ws, recompute=True)

    def keep_none():
        tps.mlp_shard_fwd(shard.X, shard.A, shard.b1, shard.B, tp_size=p, save_z=False, out=o)
        tps.mlp_shard_bwd(shard.X, shard.A, shard.B, None, None, shard.dY, tp_size=p, want_db2=True,
                          out=shard.bwd_out, workspace=ws, recompute=True, b1_i=shard.b1)

    forms = (("saved_Z_and_H", shard.mlp_step), ("saved_Z_recompute_H", keep_z),
             ("saved_none_recompute_fc1", keep_none))
    for _, fn in forms:
        for _ in range(warmup):
            fn()
    ms = {name: [] for name, _ in forms}
    for _ in range(pairs):
        for name, fn in forms:
            ms[name].append(time_stats(torch, fn, steps, 2)["mean"])
    base = ms["saved_Z_and_H"]
    act = wm.T * wm.f * 2
    med = lambda v: sorted(v)[len(v) // 2] if len(v) % 2 else 0.5 * sum(sorted(v)[len(v) // 2 - 1:len(v) // 2 + 1])  # noqa: E731,E501
    out = {"rounds": pairs, "steps_per_round": steps,
           "saved_Z_and_H": {"ms_median": round(med(base), 4), "ms_range": [round(min(base), 4), round(max(base), 4)],
                             "kept_bytes": 2 * act}}
    for name, kept in (("saved_Z_recompute_H", act), ("saved_none_recompute_fc1", 0)):
        ov = [100.0 * (a / b - 1.0) for a, b in zip(ms[name], base)]
        out[name] = {"ms_median": round(med(ms[name]), 4), "kept_bytes": kept,
                     "overhead_pct_median": round(med(ov), 2),
                     "overhead_pct_range": [round(min(ov), 2), round(max(ov), 2)]}
    return out


def run_nt_compare(torch, device, steps):
    """The step's two hardest data-gradient products, QKV dX (8192 x 12288,
    K = 4608) and the MLP dH with GeLU' (2048 x 6144, K = 12288), through this
    library and through torch.mm (hipBLASLt) on the same operands, `steps`
    times each: a fixed workload for kernel traces and hardware counters."""
    import tensor_transformer_mlp_shard_amd as tps

    g = torch.Generator(device=device).manual_seed(7)
    rn = lambda *s, sc=1.0: (torch.randn(*s, device=device, generator=g) * sc).to(torch.bfloat16)  # noqa: E731
    Xq, Wq, dQ = rn(8192, 12288), rn(12288, 4608, sc=0.006), rn(8192, 4608)
    X, A, B, Z, H, dY = (rn(2048, 12288), rn(12288, 6144, sc=0.006), rn(6144, 12288, sc=0.006), rn(2048, 6144),
                         rn(2048, 6144), rn(2048, 12288))
    out1 = torch.empty(8192, 12288, dtype=torch.bfloat16, device=device)
    out2 = torch.empty(2048, 6144, dtype=torch.bfloat16, device=device)
    for _ in range(steps):
        tps.column_linear_bwd(Xq, Wq, dQ, tp_size=8, want_db=False)
        torch.mm(dQ, Wq.t(), out=out1)
        tps.mlp_shard_bwd(X, A, B, Z, H, dY, tp_size=8, want_db1=False)
        torch.mm(dY, B.t(), out=out2)
    torch.cuda.synchronize()


def time_stats(torch, fn, steps, warmup):
    """Run `warmup` untimed calls, then exactly `steps` timed ones between two
    synchronisations.  HIP events on the current stream bracket every call, so
    besides the mean over the whole region (total time / steps) the median and
    minimum per-call times are known.  Returns dict(mean, median, min, wall)
    in ms per call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    median = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return {"mean": ev[0].elapsed_time(ev[steps]) / steps, "median": median, "min": per[0],
            "wall": wall * 1e3 / steps}


def time_steps(torch, fn, steps, warmup):
    st = time_stats(torch, fn, steps, warmup)
    return st["mean"], st["wall"]


def _rates(flop, st):
    """TFLOP/s and % of the bf16 peak from the median, plus mean / median / min ms."""
    tf = flop / (st["median"] * 1e-3) / 1e12
    return {"ms_mean": round(st["mean"], 4), "ms_median": round(st["median"], 4), "ms_min": round(st["min"], 4),
            "tflops": round(tf, 1), "pct_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2)}


def roofline_from_trace(tps, torch, fn, steps):
    """Per-kernel HIP-event times over `steps` steps (the library brackets each
    launch on its own stream); returns (dominant kernel entry, all entries)."""
    tps.trace_start(4096)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    kernels = tps.trace_stop()
    dom = max(kernels, key=lambda k: k["total_ms"])
    return dom, kernels


def _source_hash():
    h = hashlib.sha256()
    for name in ("gemm_bf16.hip", "gemm.h", "common.h", "lds_dma.h", "gelu.h"):
        with open(os.path.join(ROOT, "tensor_transformer_mlp_shard_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, launches):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    ent = data.get("kernels", {}).get(kernel)
    if not ent or data.get("source_hash") != _source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(shard, frac_tokens=1):
    """The fp64 oracle timed on 1/frac_tokens of each part's tokens (same
    weights, same formulas) on this host."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    f64 = lambda t: t.to(dtype=shard.torch.float64).numpy()  # noqa: E731
    m, a = shard.host_mlp, shard.host_attn
    Tm = shard.wm.T // frac_tokens
    Ta = shard.wa.T // frac_tokens
    X, A, b1, B, dY = f64(m["X"][:Tm]), f64(m["A"]), f64(m["b1"]), f64(m["B"]), f64(m["dY"][:Tm])
    Xa, Wq, bq, O, Wo, dQ, dYa = (f64(a["X"][:Ta]), f64(a["W_qkv"]), f64(a["b_qkv"]), f64(a["O"][:Ta]),
                                 f64(a["W_o"]), f64(a["dQKV"][:Ta]), f64(a["dY"][:Ta]))
    t0 = time.perf_counter()
    oracle.mlp_shard_fwd(X, A, b1, B)
    r = oracle.mlp_shard_bwd(X, A, b1, B, dY)
    oracle.bias_grad(dY)
    oracle.column_linear_fwd(Xa, Wq, bq)
    oracle.linear_bwd(Xa, Wq, dQ)
    oracle.row_linear_fwd(O, Wo)
    oracle.linear_bwd(O, Wo, dYa)
    dt = time.perf_counter() - t0
    del r
    flops = _flops_mlp(Tm, shard.wm.h, shard.wm.f) + _flops_attn(Ta, shard.wa.h, shard.wa.F // shard.wa.tp,
                                                                 shard.wa.h // shard.wa.tp)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle, one step on 1/{frac_tokens} of the tokens "
                      f"(MLP T={Tm}, attention T={Ta}; full weights): {flops:.3e} FLOP in {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-frac", type=int, default=1, help="oracle sample = 1/N of the tokens")
    ap.add_argument("--part", choices=["all", "mlp", "attn", "core_attn", "sp_edge", "side", "nt_compare"],
                    default="all",
                    help="run only one part (for profiling runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the step (the other workloads, selective recompute, "
                         "core attention, sequence-parallel edge, ...): for profiler runs whose per-kernel "
                         "averages must be the step's")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this many MiB, three times (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU's shard; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path: run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from tensor_transformer_mlp_shard_amd import _native

    if not os.path.exists(_native.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    device = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.part == "core_attn":
        print(json.dumps({"core_attention": measure_core_attention(torch, device, args.steps, args.warmup)}),
              flush=True)
        return
    if args.part == "sp_edge":
        print(json.dumps({"sp_edge": measure_sp_edge(torch, device, args.steps, args.warmup)}), flush=True)
        return
    if args.part == "side":
        print(json.dumps({"side_kernels": measure_side(torch, device, args.steps, args.warmup)}), flush=True)
        return
    if args.part == "nt_compare":
        run_nt_compare(torch, device, args.steps)
        print(json.dumps({"nt_compare": "done", "steps": args.steps}), flush=True)
        return
    shard = Shard(device)
    fn = {"all": shard.step, "mlp": shard.mlp_step, "attn": shard.attn_step}[args.part]
    flops = {"all": shard.flops_mlp + shard.flops_attn, "mlp": shard.flops_mlp, "attn": shard.flops_attn}[args.part]

    st = time_stats(torch, fn, args.steps, args.warmup)
    ms, wall_ms = st["mean"], st["wall"]
    value = flops / (ms * 1e-3) / 1e12
    configs = {}
    if args.part == "all" and not args.no_extras:
        configs = measure_configs(torch, device, shard, min(args.steps, 50), min(args.warmup, 20))

    dom, kernels = roofline_from_trace(shard.tps, torch, fn, args.steps)
    avg_ms = dom["total_ms"] / dom["launches"]
    if dom["flops"] > 0:
        achieved = dom["flops"] / dom["launches"] / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = dom["bytes"] / dom["launches"] / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic_for(dom["name"], dom["launches"])
    roof["kernel"] = dom["name"]
    roof["launches_per_step"] = dom["launches"] // args.steps
    roof["avg_launch_ms"] = round(avg_ms, 5)
    # what the matrix cores sustain with no memory traffic under the same power limit
    shard.tps.mfma_probe(iters=20000)
    probe = shard.tps.mfma_probe(iters=100000)
    if roof["bound"] == "mfma":
        roof["frac_of_mfma_probe"] = round(achieved / probe["tflops"], 4)
    kern = [{"name": k["name"], "launches_per_step": k["launches"] // args.steps,
             "ms_per_step": round(k["total_ms"] / args.steps, 4),
             "tflops": round(k["flops"] / (k["total_ms"] * 1e-3) / 1e12, 1) if k["flops"] else None,
             "gbs": round(k["bytes"] / (k["total_ms"] * 1e-3) / 1e9, 1)} for k in kernels]

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(st["median"], 4),
        "ms_per_step_min": round(st["min"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normals, random-init weights)",
        "config": {
            "workload": ("175B-shaped TP=8 layer shard, one rank: MLP T=2048 h=12288 f=6144 fwd+bwd "
                         "+ attention linears T=8192 QKV 12288->4608 (bias) and out-proj 1536->12288 fwd+bwd"
                         if args.part == "all" else f"part={args.part}"),
            "tp": 8,
            "flop_per_step": flops,
        },
        "pct_of_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "wall_ms_per_step": round(wall_ms, 4),
        "configs": configs,
        "roofline": roof,
        "mfma_probe": {"tflops": round(probe["tflops"], 1), "clock_ghz": round(probe["clock_ghz_mean"], 3),
                       "mfma_busy": round(probe["mfma_busy"], 3), "compute_units": probe["compute_units"],
                       "note": "register-only bf16 MFMA stream on random operands, no memory traffic"},
        "kernels": kern,
    }
    if args.part == "all" and not args.no_extras:
        sh16 = Shard(device, "fp16")
        ms16, _ = time_steps(torch, sh16.step, min(args.steps, 50), min(args.warmup, 10))
        out["fp16_step"] = {"ms": round(ms16, 4), "tflops": round(flops / (ms16 * 1e-3) / 1e12, 2),
                            "note": "the same step with IEEE-half storage (fp16 matrix-core instruction)"}
        del sh16
        out["sp_edge"] = measure_sp_edge(torch, device, min(args.steps, 50), min(args.warmup, 10))
        out["side_kernels"] = measure_side(torch, device, min(args.steps, 50), min(args.warmup, 10))
        out["selective_recompute"] = measure_recompute(torch, shard, min(args.steps, 50), min(args.warmup, 10))
        out["core_attention"] = measure_core_attention(torch, device, min(args.steps, 50), min(args.warmup, 10))
        out["vendor_gemms"] = measure_vendor_gemms(torch, shard, min(args.steps, 50), min(args.warmup, 10))
    if not args.no_cpu_baseline and args.part == "all":
        out["cpu_baseline"] = cpu_baseline(shard, args.cpu_frac)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
