"""Tensor-parallel shard emulation on one GPU: every rank of a TP group runs
its shard through the C ABI, the host combines the partials the way the
collectives would, and the result must equal the unsharded layer computed by
the fp64 oracle.

The combinations are the ones the pages give for the two shard kinds
("Megatron-LM：NVIDIA 的大规模并行训练方案", 张量并行原理; "分布式训练基础…",
2.2 核心原理): the column-parallel outputs concatenate along the features
(Y = [X A_1, ..., X A_p]), the row-parallel partials sum (Y = sum_i X_i B_i,
AllReduce).  The backward mirrors them: the column-parallel input gradient
dX = sum_i dX_i, the parameter gradients of a column shard concatenate along
the columns and those of a row shard along the rows; the row-parallel output
bias gradient is computed once from the replicated dY.

Workloads: the tiny TP=2 MLP (fp32, 1e-5), the GPT h=1024 TP=2 MLP shard, and
the 175B TP=8 MLP shard and attention-linear shards scaled down in tokens and
width with the TP degree kept at 8 (bf16 and fp16, 5e-3)."""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_shard_amd as tps
from tensor_transformer_mlp_shard_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"fp32": 1e-5, "bf16": 5e-3, "fp16": 5e-3}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _col(t, p, i):
    """Rank i's contiguous block of the last dimension (column-parallel shard)."""
    w = t.shape[-1] // p
    return t[..., i * w:(i + 1) * w].contiguous()


def _row(t, p, i):
    """Rank i's contiguous block of rows (row-parallel shard)."""
    w = t.shape[0] // p
    return t[i * w:(i + 1) * w].contiguous()


def _rel(name, got, ref, tol):
    e = oracle.rel_fro(got, ref)
    print(f"  {name:10s} rel_fro={e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: rel_fro {e:.3e} > {tol:g}"


MLP_CASES = [  # (T, h, F, p, dtype, sigma_w, seed)
    (128, 256, 1024, 2, "fp32", 0.02, 1235),      # the tiny TP=2 workload's shapes
    (4096, 1024, 4096, 2, "bf16", 0.02, 1236),    # GPT h=1024, TP=2 (whole layer)
    (384, 1536, 6144, 8, "bf16", 0.006, 1238),    # 175B MLP at TP=8, h and tokens / 8
    (384, 1536, 6144, 8, "fp16", 0.006, 1238),
]


@pytest.mark.parametrize("case", MLP_CASES, ids=[f"T{c[0]}_h{c[1]}_F{c[2]}_p{c[3]}_{c[4]}" for c in MLP_CASES])
def test_mlp_ranks_combine_to_unsharded_layer(case):
    T, h, F, p, dt, sw, seed = case
    tol = TOL[dt]
    d = synth.mlp_inputs(T, h, F, p, dt, sw, seed=seed, full=True)
    X, dY = d["X"].to(DEV), d["dY"].to(DEV)
    print(f"MLP shard emulation T={T} h={h} F={F} p={p} {dt}", flush=True)
    Y = dX = db2 = None
    dA, dB, db1 = [], [], []
    for i in range(p):
        A_i = _col(d["A"], p, i).to(DEV)
        b1_i = _col(d["b1"], p, i).to(DEV)
        B_i = _row(d["B"], p, i).to(DEV)
        Z, H, Y_i = tps.mlp_shard_fwd(X, A_i, b1_i, B_i, tp_size=p)
        g = tps.mlp_shard_bwd(X, A_i, B_i, Z, H, dY, tp_size=p, want_db2=True)
        torch.cuda.synchronize()
        Y = f64(Y_i) if Y is None else Y + f64(Y_i)          # row-parallel AllReduce
        dX = f64(g["dX"]) if dX is None else dX + f64(g["dX"])  # column-parallel backward AllReduce
        dA.append(f64(g["dA"]))
        dB.append(f64(g["dB"]))
        db1.append(f64(g["db1"]))
        db2 = f64(g["db2"])                                   # replicated: the same on every rank
    x, a, bb1, bb, dy = (f64(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    _, _, Y_ref = oracle.mlp_shard_fwd(x, a, bb1, bb)
    ref = oracle.mlp_shard_bwd(x, a, bb1, bb, dy)
    _rel("sum Y_i", Y, Y_ref, tol)
    _rel("sum dX_i", dX, ref["dX"], tol)
    _rel("[dA_i]", np.concatenate(dA, axis=1), ref["dA"], tol)
    _rel("[dB_i]", np.concatenate(dB, axis=0), ref["dB"], tol)
    _rel("[db1_i]", np.concatenate(db1), ref["db1"], tol if dt != "fp32" else 1e-5)
    _rel("db2", db2, oracle.bias_grad(dy), tol if dt != "fp32" else 1e-5)


LINEAR_CASES = [  # (T, h, p, dtype): 175B attention linears scaled down, QKV width 3 h
    (512, 1536, 8, "bf16"),
    (520, 1536, 8, "fp16"),
    (257, 1024, 2, "bf16"),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=[f"T{c[0]}_h{c[1]}_p{c[2]}_{c[3]}" for c in LINEAR_CASES])
def test_attention_linear_ranks_combine_to_unsharded_layer(case):
    T, h, p, dt = case
    tol = TOL[dt]
    g = synth.seeded(T * 31 + h + p)
    X = synth.randn(g, (T, h), 1.0, dt)
    Wq = synth.randn(g, (h, 3 * h), 0.02, dt)
    bq = synth.randn(g, (3 * h,), 0.02, dt)
    O = synth.randn(g, (T, h), 1.0, dt)
    Wo = synth.randn(g, (h, h), 0.02, dt)
    bo = synth.randn(g, (h,), 0.02, dt)
    dQ = synth.randn(g, (T, 3 * h), 1.0, dt)
    dY = synth.randn(g, (T, h), 1.0, dt)
    print(f"attention-linear shard emulation T={T} h={h} p={p} {dt}", flush=True)
    Xd, dYd = X.to(DEV), dY.to(DEV)
    Q, dXq, dWq, dbq = [], None, [], []
    Yo, dO, dWo, dbo = None, [], [], None
    for i in range(p):
        Wq_i = _col(Wq, p, i).to(DEV)
        bq_i = _col(bq, p, i).to(DEV)
        dQ_i = _col(dQ, p, i).to(DEV)
        O_i = _col(O, p, i).to(DEV)
        Wo_i = _row(Wo, p, i).to(DEV)
        # QKV column shard
        Q.append(f64(tps.column_linear(Xd, Wq_i, bq_i, tp_size=p)))
        gq = tps.column_linear_bwd(Xd, Wq_i, dQ_i, tp_size=p)
        # output projection row shard; its bias on rank 0 only
        Yo_i = tps.row_linear(O_i, Wo_i, bo.to(DEV) if i == 0 else None, tp_size=p)
        go = tps.row_linear_bwd(O_i, Wo_i, dYd, tp_size=p, want_db=(i == 0))
        torch.cuda.synchronize()
        dXq = f64(gq["dX"]) if dXq is None else dXq + f64(gq["dX"])
        dWq.append(f64(gq["dW"]))
        dbq.append(f64(gq["db"]))
        Yo = f64(Yo_i) if Yo is None else Yo + f64(Yo_i)
        dO.append(f64(go["dX"]))
        dWo.append(f64(go["dW"]))
        if i == 0:
            dbo = f64(go["db"])
    x, wq, b_q, o, wo, b_o, dq, dy = (f64(t) for t in (X, Wq, bq, O, Wo, bo, dQ, dY))
    _, Q_ref = oracle.column_linear_fwd(x, wq, b_q)
    rq = oracle.linear_bwd(x, wq, dq)
    _rel("[QKV_i]", np.concatenate(Q, axis=1), Q_ref, tol)
    _rel("sum dX_i", dXq, rq["dX"], tol)
    _rel("[dWqkv_i]", np.concatenate(dWq, axis=1), rq["dW"], tol)
    _rel("[dbqkv_i]", np.concatenate(dbq), rq["db"], 1e-5)
    _rel("sum Yo_i", Yo, oracle.row_linear_fwd(o, wo, b_o), tol)
    ro = oracle.linear_bwd(o, wo, dy)
    _rel("[dO_i]", np.concatenate(dO, axis=1), ro["dX"], tol)
    _rel("[dWo_i]", np.concatenate(dWo, axis=0), ro["dW"], tol)
    _rel("dbo", dbo, ro["db"], 1e-5)
