"""Every 16-bit store of the GPU path rounds to nearest-even.

The pages' mixed-precision training keeps fp32 master weights and 16-bit
activations ("课程导入" §1.4.1); the reading taken here is fp32 arithmetic with
one round-to-nearest-even conversion per stored element.  A truncating or
round-half-away store still passes the Frobenius tolerances of the parity
tests (it only doubles the rounding error), so this test crafts inputs whose
fp32 results sit exactly halfway between two neighbouring bf16 (or fp16)
values, and compares the stored bits with torch's host RNE conversion of the
oracle's exact fp64 value.

Construction: output element (t, n) = x1_t + hu_t * s_n, where x1_t is a
16-bit value of either sign with magnitude in [1/16, 16), hu_t is half the
16-bit spacing at x1_t, and s_n cycles over +-1 and +-3 (ties: halfway
between two neighbours, resolved by the even mantissa) and +-1/2, +-3/2 (not
ties).  Every such sum is exact in fp32, so the kernel's fp32 result is the
oracle's value and the only rounding is the store.
  * GEMM STORE epilogue: X[t] = (x1_t, hu_t, 0...), W[0] = 1, W[1] = s
    (row-parallel linear, and column-parallel with a zero bias), on small
    ragged tiles and on the 256 x 384 tiles of the 175B shard shape.
  * GEMM bias + GeLU epilogue: the saved pre-activation Z.
  * GEMM GeLU' epilogue: dH = dY B^T built the same way, Z = 8 everywhere
    (GeLU'(8) = 1 + 4e-14, i.e. exactly 1 in the fp32 product the kernel and
    the expected value both form), A = I so that dX = dZ A^T = dZ.
  * LayerNorm forward with rows of alternating +-1 (mean 0, rstd 1, eps = 0):
    y = +-gamma + beta with gamma = x1, beta = hu * s.
  * bias + dropout + residual with p = 0: out = residual + y + b."""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_shard_amd as tps

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
MANT = {"bf16": 7, "fp16": 10}        # stored mantissa bits
SIGMAS = np.array([1.0, -1.0, 3.0, -3.0, 0.5, -0.5, 1.5, -1.5])


def _x1_hu(n, dt, seed):
    """n 16-bit values x1 (either sign, magnitude in [1/16, 16)) and half the
    16-bit spacing at each of them, as float64."""
    rng = np.random.default_rng(seed)
    mb = MANT[dt]
    e = rng.integers(-4, 4, n)
    m = rng.integers(0, 2 ** mb, n)
    m[:4] = [0, 2 ** mb - 1, 0, 2 ** mb - 1]     # binade edges
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    x1 = sign * (1.0 + m / 2.0 ** mb) * np.exp2(e)
    hu = np.exp2(e - mb - 1.0)
    return x1, hu


def _tie_fraction(x, dt):
    """Fraction of the values that lie exactly halfway between two 16-bit neighbours."""
    a = np.abs(x)
    u = np.exp2(np.floor(np.log2(a)) - MANT[dt])
    frac = (a / u) % 1.0
    return float(np.mean(frac == 0.5))


def _t(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to(TORCH_DT[dt])


def _expect_bits(exact, dt):
    """Host RNE of the exact value (exact in fp32 by construction)."""
    f32 = torch.from_numpy(np.ascontiguousarray(exact)).to(torch.float32)
    assert np.array_equal(f32.double().numpy(), exact), "the crafted value is not exact in fp32"
    return f32.to(TORCH_DT[dt]).view(torch.int16)


def _assert_bits(name, got, exact, dt):
    want = _expect_bits(exact, dt)
    bad = int((got.detach().cpu().view(torch.int16) != want).sum())
    ties = _tie_fraction(exact, dt)
    print(f"  {name:18s} {dt}: {exact.size} stores, {ties:.0%} exact ties, {bad} mismatches", flush=True)
    assert ties >= 0.3, "the fixture must exercise ties"
    assert bad == 0


def _gemm_operands(T, N, dt, seed):
    x1, hu = _x1_hu(T, dt, seed)
    X = np.zeros((T, 8))
    X[:, 0], X[:, 1] = x1, hu
    W = np.zeros((8, N))
    W[0] = 1.0
    W[1] = np.resize(SIGMAS, N)
    return X, W


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("T,N", [(300, 392), (2048, 12288)], ids=["ragged", "256x384"])
def test_store_epilogue_rounds_to_even(dt, T, N):
    print(f"RNE store T={T} N={N} {dt}", flush=True)
    X, W = _gemm_operands(T, N, dt, 100 + T)
    Xd, Wd = _t(X, dt).to(DEV), _t(W, dt).to(DEV)
    y_row = tps.row_linear(Xd, Wd, None, tp_size=1)
    y_col = tps.column_linear(Xd, Wd, torch.zeros(N, dtype=TORCH_DT[dt], device=DEV), tp_size=1)
    torch.cuda.synchronize()
    _assert_bits("row_linear Y", y_row, oracle.row_linear_fwd(X, W), dt)
    _assert_bits("column_linear Y", y_col, oracle.column_linear_fwd(X, W, np.zeros(N))[1], dt)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_bias_gelu_epilogue_stores_z_rounded_to_even(dt):
    T, N = 300, 392
    print(f"RNE bias+GeLU Z T={T} N={N} {dt}", flush=True)
    X, W = _gemm_operands(T, N, dt, 7)
    y, z = tps.column_linear(_t(X, dt).to(DEV), _t(W, dt).to(DEV), torch.zeros(N, dtype=TORCH_DT[dt], device=DEV),
                             tp_size=1, act="gelu", save_z=True)
    torch.cuda.synchronize()
    Z_ref, H_ref = oracle.column_linear_fwd(X, W, np.zeros(N), act="gelu")
    _assert_bits("column_linear Z", z, Z_ref, dt)
    assert oracle.rel_fro(y.double().cpu().numpy(), H_ref) <= 5e-3


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_dgelu_epilogue_rounds_to_even(dt):
    T, h = 300, 136
    f = h
    print(f"RNE GeLU' dZ T={T} h=f={h} {dt}", flush=True)
    x1, hu = _x1_hu(T, dt, 11)
    dY = np.zeros((T, h))
    dY[:, 0], dY[:, 1] = x1, hu
    B = np.zeros((f, h))                  # B_i [f x h]: dH[t, j] = dY[t, 0] + dY[t, 1] s_j
    B[:, 0] = 1.0
    B[:, 1] = np.resize(SIGMAS, f)
    A = np.eye(h, f)                      # dX = dZ A^T = dZ
    X = np.zeros((T, h))
    b1 = np.full(f, 8.0)                  # Z = X A + b1 = 8 everywhere (the saved pre-activation)
    Z = np.full((T, f), 8.0)
    d = {k: _t(v, dt).to(DEV) for k, v in (("X", X), ("A", A), ("B", B), ("Z", Z), ("dY", dY))}
    Hd = torch.zeros((T, f), dtype=TORCH_DT[dt], device=DEV)
    g = tps.mlp_shard_bwd(d["X"], d["A"], d["B"], d["Z"], Hd, d["dY"], tp_size=1)
    torch.cuda.synchronize()
    # The oracle's dZ = dH * GeLU'(8) with GeLU'(8) = 1 + 4e-14; the kernel forms the
    # product in fp32, where that factor is 1.  Both sides take the rounding
    # decision from the same fp32 value: the oracle's dZ rounded to fp32 (= dH).
    ref = oracle.mlp_shard_bwd(X, A, b1, B, dY)
    assert np.all(ref["Z"] == 8.0)
    assert float(np.float32(oracle.gelu_grad(8.0))) == 1.0
    dz32 = ref["dZ"].astype(np.float32).astype(np.float64)
    _assert_bits("mlp_bwd dZ (as dX)", g["dX"], dz32, dt)
    # and the non-tie part of the oracle comparison holds as usual
    assert oracle.rel_fro(g["dX"].double().cpu().numpy(), ref["dX"]) <= 5e-3


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_layernorm_fwd_rounds_to_even(dt):
    rows, h = 64, 1024
    print(f"RNE LayerNorm rows={rows} h={h} {dt}", flush=True)
    X = np.where((np.arange(rows)[:, None] + np.arange(h)[None, :]) % 2 == 0, 1.0, -1.0)
    gamma, hu = _x1_hu(h, dt, 21)
    beta = hu * np.resize(SIGMAS, h)
    y, mean, rstd = tps.layernorm_fwd(_t(X, dt).to(DEV), _t(gamma, dt).to(DEV), _t(beta, dt).to(DEV), eps=0.0)
    torch.cuda.synchronize()
    # the construction needs the kernel's statistics exact: mean 0 and 1/sqrt(var) = 1
    assert torch.all(mean == 0).item() and torch.all(rstd == 1).item()
    Y_ref, _, _ = oracle.layernorm_fwd(X, gamma, beta, eps=0.0)
    _assert_bits("layernorm_fwd Y", y, Y_ref, dt)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_bias_dropout_add_rounds_to_even(dt):
    rows, h = 96, 1032
    print(f"RNE bias+dropout+residual rows={rows} h={h} {dt}", flush=True)
    x1, hu = _x1_hu(rows * h, dt, 31)
    R = x1.reshape(rows, h)
    Y = (hu * np.resize(SIGMAS, rows * h)).reshape(rows, h)
    out = tps.bias_dropout_add_fwd(_t(Y, dt).to(DEV), torch.zeros(h, dtype=TORCH_DT[dt], device=DEV),
                                   _t(R, dt).to(DEV), p=0.0, seed=3, offset=0)
    torch.cuda.synchronize()
    ref, keep = oracle.bias_dropout_add_fwd(Y, np.zeros(h), R, 0.0, 3, 0)
    assert keep.all()
    _assert_bits("bias_dropout_add", out, ref, dt)
