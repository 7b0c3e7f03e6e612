"""GPU parity of the K-split weight gradient: a dW = X^T dY [M x N] whose tiles
would fill at most half of the CUs is computed by twice the workgroups, each
half of the contraction, the second half's fp32 partial added to dW by a second
pass in a fixed order.  It runs where the workspace has room for the partial
(always in the MLP backward; in the linear backwards when a workspace is
passed).  Checked against the oracle with the contraction ragged against the
32-deep K step and split into unequal halves (65 steps), with and without the
bias gradient riding along, with accumulate, unsplit (no workspace) against
split, and bitwise repeatable."""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_shard_amd as tps
from tensor_transformer_mlp_shard_amd import _native, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 5e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV) if isinstance(a, np.ndarray) else a.to(DEV)


def _rel(name, got, ref, tol=TOL):
    e = oracle.rel_fro(got, ref)
    print(f"  {name:8s} rel_fro={e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: rel_fro {e:.3e} > {tol:g}"


# (T, K, N, p): dW is [K x N/p] (column) or [K/p x N] (row); T = 2080 is 65 K steps of 32
CASES = [(2080, 512, 640, 1), (2080, 1024, 2048, 2), (4096, 256, 1024, 4)]


@pytest.mark.parametrize("T,K,N,p", CASES, ids=[f"T{c[0]}_K{c[1]}_N{c[2]}_p{c[3]}" for c in CASES])
def test_ksplit_linear_bwd(T, K, N, p):
    print(f"case T={T} K={K} N={N} p={p}", flush=True)
    g = synth.seeded(T + K + N + p)
    X = synth.randn(g, (T, K), 1.0, "bf16")
    W = synth.randn(g, (K, N // p), 0.05, "bf16")
    dY = synth.randn(g, (T, N // p), 1.0, "bf16")
    Xi = synth.randn(g, (T, K // p), 1.0, "bf16")
    Wr = synth.randn(g, (K // p, N), 0.05, "bf16")
    dYr = synth.randn(g, (T, N), 1.0, "bf16")
    gc = tps.column_linear_bwd(dev(X), dev(W), dev(dY), tp_size=p)                  # split (workspace)
    gc0 = tps.column_linear_bwd(dev(X), dev(W), dev(dY), tp_size=p, want_db=False)  # no workspace: unsplit
    gr = tps.row_linear_bwd(dev(Xi), dev(Wr), dev(dYr), tp_size=p)
    torch.cuda.synchronize()
    rc = oracle.linear_bwd(f64(X), f64(W), f64(dY))
    _rel("col.dW", f64(gc["dW"]), rc["dW"])
    _rel("col.db", f64(gc["db"]), rc["db"], 1e-5)
    _rel("col.dW0", f64(gc0["dW"]), rc["dW"])
    # the two forms differ only in where fp32 rounding falls
    _rel("split~0", f64(gc["dW"]), f64(gc0["dW"]), 1e-5)
    rr = oracle.linear_bwd(f64(Xi), f64(Wr), f64(dYr))
    _rel("row.dW", f64(gr["dW"]), rr["dW"])
    _rel("row.db", f64(gr["db"]), rr["db"], 1e-5)


def test_ksplit_accumulate_and_repeat():
    T, K, N = 2080, 512, 640
    g = synth.seeded(77)
    X, W, dY = (dev(synth.randn(g, s, sg, "bf16")) for s, sg in (((T, K), 1.0), ((K, N), 0.05), ((T, N), 1.0)))
    g1 = tps.column_linear_bwd(X, W, dY, tp_size=1)
    g2 = tps.column_linear_bwd(X, W, dY, tp_size=1)
    base = {k: torch.full_like(g1[k], 0.5) for k in ("dW", "db")}
    acc = {k: v.clone() for k, v in base.items()}
    tps.column_linear_bwd(X, W, dY, tp_size=1, accumulate=True, out=acc)
    torch.cuda.synchronize()
    assert torch.equal(g1["dW"], g2["dW"]) and torch.equal(g1["db"], g2["db"])
    # dW with accumulate is (old + first half) + second half: fp32 roundings at
    # the size of the half sums, which may exceed the result where they cancel
    e = float((acc["dW"] - (base["dW"] + g1["dW"])).abs().max())
    bound = 16 * 2.0 ** -24 * (float(g1["dW"].abs().max()) + 0.5)
    print(f"  dW accumulate max|diff| {e:.3e} (bound {bound:.3e})", flush=True)
    assert e <= bound
    torch.testing.assert_close(acc["db"], base["db"] + g1["db"], rtol=1e-6, atol=1e-6)


def test_ksplit_mlp_bwd_against_oracle():
    """MLP backward at a shape whose two weight gradients split (128 x 128 tiles,
    under half of the CUs), db1 and db2 riding along, against the oracle."""
    T, h, F, p = 2080, 384, 1536, 2
    d = synth.mlp_inputs(T, h, F, p, "bf16", 0.05, seed=91, full=False)
    Xd, Ad, b1d, Bd, dYd = (dev(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    Z, H, _ = tps.mlp_shard_fwd(Xd, Ad, b1d, Bd, tp_size=p)
    gb = tps.mlp_shard_bwd(Xd, Ad, Bd, Z, H, dYd, tp_size=p, want_db2=True)
    torch.cuda.synchronize()
    ref = oracle.mlp_shard_bwd(f64(d["X"]), f64(d["A"]), f64(d["b1"]), f64(d["B"]), f64(d["dY"]))
    ref["db2"] = oracle.bias_grad(f64(d["dY"]))
    for k, tol in (("dX", TOL), ("dA", TOL), ("dB", TOL), ("db1", TOL), ("db2", 1e-5)):
        _rel(k, f64(gb[k]), ref[k], tol)
