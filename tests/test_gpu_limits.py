"""GPU parity at the size limits of the C ABI.

* A column-parallel linear with T = 393216 tokens and K = 8192 (a 6.4 GB
  input: byte offsets past 2^32, a 393216-long contraction in the weight
  gradient and the bias-gradient sums).  dY is zero except on sampled rows, so
  dW = X[R]^T dY[R] and db = sum over R are exact reductions the oracle can
  evaluate from the sampled rows; the zero rows of dX must be exactly zero.
* Feature dimensions at the 2^21 limit (K and N in turn)."""
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


def _rel(name, got, ref, tol=TOL):
    e = oracle.rel_fro(got, ref)
    print(f"  {name:8s} rel_fro={e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: rel_fro {e:.3e} > {tol:g}"


def test_column_linear_past_4gib_offsets():
    T, K, N = 393216, 8192, 512
    print(f"large linear T={T} K={K} N={N}", flush=True)
    X = synth.device_randn((T, K), 1.0, "bf16", 2001, DEV)
    W = synth.device_randn((K, N), 0.02, "bf16", 2002, DEV)
    b = synth.device_randn((N,), 0.02, "bf16", 2003, DEV)
    rng = np.random.default_rng(5)
    R = np.unique(np.concatenate([rng.choice(T, 40, replace=False), [0, T - 1, T // 2, (1 << 18) + 5]]))
    Rd = torch.from_numpy(R).to(DEV)
    dY = torch.zeros((T, N), dtype=torch.bfloat16, device=DEV)
    dY[Rd] = synth.device_randn((len(R), N), 1.0, "bf16", 2004, DEV)
    Y = tps.column_linear(X, W, b, tp_size=1)
    g = tps.column_linear_bwd(X, W, dY, tp_size=1)
    torch.cuda.synchronize()
    x_r, w, dy_r = f64(X[Rd]), f64(W), f64(dY[Rd])
    _, y_ref = oracle.column_linear_fwd(x_r, w, f64(b))
    _rel("Y[R]", f64(Y[Rd]), y_ref)
    ref = oracle.linear_bwd(x_r, w, dy_r)          # dW and db over the nonzero rows are the whole sums
    _rel("dX[R]", f64(g["dX"][Rd]), ref["dX"])
    _rel("dW", f64(g["dW"]), ref["dW"])
    _rel("db", f64(g["db"]), ref["db"])
    zero_rows = torch.from_numpy(np.setdiff1d(np.arange(T - 64, T), R)).to(DEV)
    assert torch.count_nonzero(g["dX"][zero_rows]).item() == 0


@pytest.mark.parametrize("K,N", [(1 << 21, 8), (8, 1 << 21)], ids=["K=2^21", "N=2^21"])
def test_feature_dim_limit(K, N):
    T = 16
    print(f"feature limit T={T} K={K} N={N}", flush=True)
    X = synth.device_randn((T, K), 1.0, "bf16", 2101 + K, DEV)
    W = synth.device_randn((K, N), 0.02, "bf16", 2102 + N, DEV)
    dY = synth.device_randn((T, N), 1.0, "bf16", 2103, DEV)
    Y = tps.column_linear(X, W, None, tp_size=1)
    g = tps.column_linear_bwd(X, W, dY, tp_size=1)
    torch.cuda.synchronize()
    x, w, dy = f64(X), f64(W), f64(dY)
    _, y_ref = oracle.column_linear_fwd(x, w, None)
    _rel("Y", f64(Y), y_ref)
    ref = oracle.linear_bwd(x, w, dy)
    _rel("dX", f64(g["dX"]), ref["dX"])
    _rel("dW", f64(g["dW"]), ref["dW"])
    _rel("db", f64(g["db"]), ref["db"])


def test_contraction_at_limit_with_384_row_panels():
    """dX = dY W^T with a 2^21-long contraction, T = 4096 and 6144 outputs, the
    shape for which the 256 x 384 tile is chosen: its weight panels hold 384
    rows 2^22 bytes apart, so their last rows sit 1.6 GB past the panel base
    and must still be read (none zero-filled).  About 90 GB of device memory."""
    T, K_in, N_out = 4096, 6144, 1 << 21
    print(f"contraction limit T={T} K={K_in} N={N_out}", flush=True)
    X = synth.device_randn((T, K_in), 1.0, "bf16", 2201, DEV)
    W = torch.empty((K_in, N_out), dtype=torch.bfloat16, device=DEV)
    for i, r0 in enumerate(range(0, K_in, 512)):      # drawn in slices to bound the fp32 temporary
        W[r0:r0 + 512] = synth.device_randn((min(512, K_in - r0), N_out), 0.02, "bf16", 2202 + i, DEV)
    dY = synth.device_randn((T, N_out), 1.0, "bf16", 2300, DEV)
    g = tps.column_linear_bwd(X, W, dY, tp_size=1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    R = np.sort(rng.choice(T, 8, replace=False))
    # output columns on rows 256..383 of their 384-row weight panel, and a few others
    J = np.sort(np.concatenate([rng.choice(np.arange(256, 384), 24, replace=False) + 384 * t for t in range(3)] +
                               [rng.choice(K_in, 24, replace=False)]))
    Rd, Jd = torch.from_numpy(R).to(DEV), torch.from_numpy(J).to(DEV)
    # dX[R, J] = dY[R] W[J]^T: the oracle's data gradient of the narrowed product
    # X[R][:, J] W[J] (each output column depends only on its own weight row)
    ref_x = oracle.linear_bwd(f64(X[Rd][:, Jd]), f64(W[Jd]), f64(dY[Rd]))
    _rel("dX[R,J]", f64(g["dX"][Rd][:, Jd]), ref_x["dX"])
    Kc = np.sort(rng.choice(N_out, 32, replace=False))
    Kd = torch.from_numpy(Kc).to(DEV)
    # dW[J, Kc] = X[:, J]^T dY[:, Kc] and db[Kc] = sum_t dY[:, Kc]: the oracle's
    # weight and bias gradients of the product narrowed to those columns
    ref_w = oracle.linear_bwd(f64(X[:, Jd]), f64(W[Jd][:, Kd]), f64(dY[:, Kd]))
    _rel("dW[J,K]", f64(g["dW"][Jd][:, Kd]), ref_w["dW"])
    _rel("db[K]", f64(g["db"][Kd]), ref_w["db"])
