"""GPU parity of the column-split launch: a product that would run as several
waves of 256 x 192 tiles (the 8192 x 4608 QKV forward) is computed as two
launches, its first columns on 256 x 384 tiles filling whole waves and the
rest on 256 x 192 tiles, every operand and output of the second part offset by
the split column.  Whole tensors against the oracle with the token count ragged
against the tile rows (T = 8100) and every epilogue that splits: bias + store
(column-parallel linear), bias + GeLU with the pre-activation saved (fc1), GeLU'
(the MLP's dZ); the split is asserted from the trace."""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_shard_amd as tps
from tensor_transformer_mlp_shard_amd import synth

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


def _traced(fn):
    tps.trace_start()
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        names = [k["name"] for k in tps.trace_stop()]
    print("  launches:", names, flush=True)
    return out, names


def _tn(dtype):
    return "bf16" if dtype == "bf16" else "f16"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_colsplit_column_linear_bias(dtype):
    # Y_i [8100 x 4608] = X W_i + b_i: 3 waves of 256 x 192 alone; split into columns
    # [0, 3072) on 256 x 384 (256 tiles) and [3072, 4608) on 256 x 192 (256 tiles)
    T, K, n = 8100, 512, 4608
    print(f"case column linear T={T} K={K} n={n} {dtype}", flush=True)
    g = synth.seeded(401)
    X = synth.randn(g, (T, K), 1.0, dtype)
    W = synth.randn(g, (K, n), 0.04, dtype)
    b = synth.randn(g, (n,), 0.5, dtype)
    Y, names = _traced(lambda: tps.column_linear(dev(X), dev(W), dev(b), tp_size=1))
    assert f"gemm_{_tn(dtype)}_nn_store_256x384+256x192" in names
    _rel("Y", f64(Y), oracle.column_linear_fwd(f64(X), f64(W), f64(b))[1])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_colsplit_mlp_fc1_and_dz(dtype):
    # fc1 (bias + GeLU, Z saved) and dZ (GeLU') are [8100 x 4608]: both split
    T, h, F, p = 8100, 256, 4608, 1
    print(f"case MLP T={T} h={h} F={F} {dtype}", flush=True)
    d = synth.mlp_inputs(T, h, F, p, dtype, 0.06, seed=419, full=False)
    Xd, Ad, b1d, Bd, dYd = (dev(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    (Z, H, Y), nf = _traced(lambda: tps.mlp_shard_fwd(Xd, Ad, b1d, Bd, tp_size=p))
    assert f"gemm_{_tn(dtype)}_nn_bias_gelu_256x384+256x192" in nf
    gb, nb = _traced(lambda: tps.mlp_shard_bwd(Xd, Ad, Bd, Z, H, dYd, tp_size=p))
    assert f"gemm_{_tn(dtype)}_nt_dgelu_256x384+256x192" in nb
    x, a, b1, bb, dy = (f64(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    Zr, Hr, Yr = oracle.mlp_shard_fwd(x, a, b1, bb)
    _rel("Z", f64(Z), Zr)
    _rel("H", f64(H), Hr)
    _rel("Y", f64(Y), Yr)
    ref = oracle.mlp_shard_bwd(x, a, b1, bb, dy)
    for k in ("dX", "dA", "dB", "db1"):
        _rel(k, f64(gb[k]), ref[k])
