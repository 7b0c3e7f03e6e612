"""GPU parity of the paired backward launch: a data gradient whose tiles would
be one wave of 256 x 192 (the MLP's dZ, the row-parallel linear's dX) runs on
256 x 384 tiles beside its backward's independent weight gradient (dB_i, dW_i)
in one launch.  Whole tensors against the oracle at shapes where the launcher
pairs (asserted from the trace), with the token count ragged against both the
tile rows of the data gradient and the 32-deep K step of the weight gradient,
in bf16 and fp16, the bias gradients riding on the weight gradients (192 x 384
tiles).  The 175B-shaped MLP shard pairs its dZ with dB_i on 256 x 384 tiles; the
sampled full-size parity test covers that pair."""
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


def tps_name(dtype):
    return "bf16" if dtype == "bf16" else "f16"


def _traced(fn):
    tps.trace_start()
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        names = [k["name"] for k in tps.trace_stop()]
    print("  launches:", names, flush=True)
    return out, names


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_pair_mlp_bwd_against_oracle(dtype):
    # dZ [1000 x 11264] (K = 1536): 236 tiles of 256 x 192 alone, 120 of 256 x 384 paired
    # (the last row and column of tiles ragged); dB_i [11264 x 1536] over T = 1000 tokens
    # (31.25 K steps, db2 riding along) beside it
    T, h, F, p = 1000, 1536, 11264, 1
    print(f"case MLP T={T} h={h} F={F} p={p} {dtype}", flush=True)
    d = synth.mlp_inputs(T, h, F, p, dtype, 0.03, seed=211, full=False)
    Xd, Ad, b1d, Bd, dYd = (dev(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    Z, H, _ = tps.mlp_shard_fwd(Xd, Ad, b1d, Bd, tp_size=p)
    gb, names = _traced(lambda: tps.mlp_shard_bwd(Xd, Ad, Bd, Z, H, dYd, tp_size=p, want_db2=True))
    assert f"gemm_{tps_name(dtype)}_pair_nt_dgelu_256x384+tn_f32_192x384" in names
    ref = oracle.mlp_shard_bwd(f64(d["X"]), f64(d["A"]), f64(d["b1"]), f64(d["B"]), f64(d["dY"]))
    ref["db2"] = oracle.bias_grad(f64(d["dY"]))
    for k, tol in (("dX", TOL), ("dA", TOL), ("dB", TOL), ("db1", TOL), ("db2", 1e-5)):
        _rel(k, f64(gb[k]), ref[k], tol)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_pair_row_linear_bwd_against_oracle(dtype):
    # dX_i [3000 x 3328] (K = 5120): 216 tiles of 256 x 192 alone, 108 of 256 x 384 paired
    # (ragged tile rows); dW_i [3328 x 5120] over T = 3000 tokens (93.75 K steps) beside it
    T, K, N, p = 3000, 3328, 5120, 1
    k = K // p
    print(f"case row linear T={T} k={k} N={N} {dtype}", flush=True)
    g = synth.seeded(307)
    Xi = synth.randn(g, (T, k), 1.0, dtype)
    Wi = synth.randn(g, (k, N), 0.02, dtype)
    dY = synth.randn(g, (T, N), 1.0, dtype)
    gr, names = _traced(lambda: tps.row_linear_bwd(dev(Xi), dev(Wi), dev(dY), tp_size=p))
    assert f"gemm_{tps_name(dtype)}_pair_nt_store_256x384+tn_f32_192x384" in names
    ref = oracle.linear_bwd(f64(Xi), f64(Wi), f64(dY))
    _rel("dX", f64(gr["dX"]), ref["dX"])
    _rel("dW", f64(gr["dW"]), ref["dW"])
    _rel("db", f64(gr["db"]), ref["db"], 1e-5)


def test_pair_accumulate_adds():
    # accumulate = 1 on the paired launches: the weight gradient beside the data
    # gradient adds its product to the fp32 values already there (dB_i of the
    # MLP, dW_i of the row linear), the bias gradients to theirs; one product is
    # deterministic, so base + product matches the eager sum of the two exactly
    T, h, F, p = 1000, 1536, 11264, 1
    print(f"case MLP accumulate T={T} h={h} F={F}", flush=True)
    d = synth.mlp_inputs(T, h, F, p, "bf16", 0.03, seed=223, full=False)
    Xd, Ad, b1d, Bd, dYd = (dev(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    Z, H, _ = tps.mlp_shard_fwd(Xd, Ad, b1d, Bd, tp_size=p)
    g1 = tps.mlp_shard_bwd(Xd, Ad, Bd, Z, H, dYd, tp_size=p, want_db2=True)
    base = {k: torch.full_like(g1[k], 0.5) for k in ("dA", "dB", "db1", "db2")}
    acc = {k: v.clone() for k, v in base.items()}
    _, names = _traced(lambda: tps.mlp_shard_bwd(Xd, Ad, Bd, Z, H, dYd, tp_size=p, want_db2=True, accumulate=True,
                                                 out=acc))
    assert "gemm_bf16_pair_nt_dgelu_256x384+tn_f32_192x384" in names
    for k in ("dA", "dB"):
        assert torch.equal(acc[k], base[k] + g1[k]), k
    for k in ("db1", "db2"):
        torch.testing.assert_close(acc[k], base[k] + g1[k], rtol=1e-6, atol=1e-6)

    T, K, N = 3000, 3328, 5120
    print(f"case row linear accumulate T={T} k={K} N={N}", flush=True)
    g = synth.seeded(311)
    Xi = dev(synth.randn(g, (T, K), 1.0, "bf16"))
    Wi = dev(synth.randn(g, (K, N), 0.02, "bf16"))
    dY = dev(synth.randn(g, (T, N), 1.0, "bf16"))
    r1 = tps.row_linear_bwd(Xi, Wi, dY, tp_size=1)
    base = {k: torch.full_like(r1[k], -0.25) for k in ("dW", "db")}
    acc = {k: v.clone() for k, v in base.items()}
    _, names = _traced(lambda: tps.row_linear_bwd(Xi, Wi, dY, tp_size=1, accumulate=True, out=acc))
    assert "gemm_bf16_pair_nt_store_256x384+tn_f32_192x384" in names
    assert torch.equal(acc["dW"], base["dW"] + r1["dW"])
    torch.testing.assert_close(acc["db"], base["db"] + r1["db"], rtol=1e-6, atol=1e-6)
