"""Pins of the fp64 sequence-parallel edge oracle (oracle/sp_edge.py):
LayerNorm by its defining invariants, an independent brute-force evaluation,
torch's float64 layer_norm and finite differences; Philox4x32-10 by the
published known-answer vectors and its bijectivity; dropout by exact special
cases, statistics and finite differences; planted mistakes one of these must
catch.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import sp_edge as sp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(s):
    return np.random.default_rng(s)


# ---------------------------------------------------------------- LayerNorm

def test_rows_are_normalised():
    X = _rng(1).standard_normal((7, 33)) * 3 + 5
    Y, mean, rstd = sp.layernorm_fwd(X, np.ones(33), None, eps=0.0)
    np.testing.assert_allclose(Y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((Y ** 2).mean(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(mean, X.mean(axis=1), rtol=1e-14)


def test_affine_and_shift_scale_invariance():
    rng = _rng(2)
    X = rng.standard_normal((5, 16))
    g, b = rng.standard_normal(16), rng.standard_normal(16)
    Y, _, _ = sp.layernorm_fwd(X, g, b, eps=0.0)
    Y1, _, _ = sp.layernorm_fwd(X, np.ones(16), None, eps=0.0)
    np.testing.assert_allclose(Y, Y1 * g + b, rtol=1e-13, atol=1e-13)
    a, c = 3.7, rng.standard_normal((5, 1))
    Y2, _, _ = sp.layernorm_fwd(a * X + c, g, b, eps=0.0)
    np.testing.assert_allclose(Y2, Y, rtol=1e-12, atol=1e-12)


def test_two_element_row_closed_form():
    a, eps = 0.3, 1e-5
    Y, mean, rstd = sp.layernorm_fwd(np.array([[a, -a]]), np.ones(2), None, eps)
    np.testing.assert_allclose(Y[0], [a / math.sqrt(a * a + eps), -a / math.sqrt(a * a + eps)], rtol=1e-15)
    assert mean[0] == 0.0


def _brute_ln(X, g, b, eps):
    out = []
    for row in X.tolist():
        m = sum(row) / len(row)
        v = sum((x - m) ** 2 for x in row) / len(row)
        r = 1.0 / math.sqrt(v + eps)
        out.append([(x - m) * r * g[j] + b[j] for j, x in enumerate(row)])
    return np.array(out)


def test_layernorm_bruteforce():
    rng = _rng(3)
    for rows, h in [(1, 1), (2, 3), (4, 8), (3, 17)]:
        X = rng.standard_normal((rows, h))
        g, b = rng.standard_normal(h), rng.standard_normal(h)
        Y, _, _ = sp.layernorm_fwd(X, g, b, 1e-5)
        np.testing.assert_allclose(Y, _brute_ln(X, g.tolist(), b.tolist(), 1e-5), rtol=1e-12, atol=1e-12)


def test_layernorm_against_torch_float64():
    rng = _rng(4)
    X = rng.standard_normal((9, 64))
    g, b = rng.standard_normal(64), rng.standard_normal(64)
    dY = rng.standard_normal((9, 64))
    Y, _, _ = sp.layernorm_fwd(X, g, b, 1e-5)
    xt, gt, bt = (torch.tensor(a, requires_grad=True) for a in (X, g, b))
    yt = torch.nn.functional.layer_norm(xt, (64,), gt, bt, 1e-5)
    np.testing.assert_allclose(Y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    yt.backward(torch.tensor(dY))
    dX, dg, db = sp.layernorm_bwd(X, g, dY, 1e-5)
    np.testing.assert_allclose(dX, xt.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def _ln_fd_err(seed=5, rows=3, h=6, eps=1e-5, step=1e-6):
    rng = _rng(seed)
    X, g, b, dY = rng.standard_normal((rows, h)), rng.standard_normal(h), rng.standard_normal(h), \
        rng.standard_normal((rows, h))
    dX, dg, db = sp.layernorm_bwd(X, g, dY, eps)
    L = lambda X_, g_, b_: float(np.sum(dY * sp.layernorm_fwd(X_, g_, b_, eps)[0]))  # noqa: E731
    errs = []
    for arr, grad in ((X, dX), (g, dg), (b, db)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(*arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += step
            a2[idx] -= step
            args1 = [a1 if arr is t else t for t in (X, g, b)]
            args2 = [a2 if arr is t else t for t in (X, g, b)]
            num[idx] = (L(*args1) - L(*args2)) / (2 * step)
        errs.append(np.linalg.norm(grad - num) / np.linalg.norm(num))
    return max(errs)


def test_layernorm_finite_differences():
    assert _ln_fd_err() < 1e-7


# ---------------------------------------------------------------- Philox / dropout

def _kat():
    rows = []
    for line in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")):
        if line.strip() and not line.startswith("#"):
            w = [int(x, 16) for x in line.split()]
            rows.append((w[:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    kat = _kat()
    assert len(kat) == 3
    for ctr, key, out in kat:
        assert [int(v) for v in sp.philox4x32_10(ctr, key)] == out


def test_philox_is_a_bijection_on_a_counter_range():
    n = 1 << 15
    ctr = np.stack([np.arange(n), np.zeros(n), np.zeros(n), np.zeros(n)], axis=-1).astype(np.uint64)
    out = sp.philox4x32_10(ctr, (12345, 678))
    as_int = out.astype(np.uint64)
    packed = (as_int[:, 0] << np.uint64(32)) | as_int[:, 1]
    assert len(np.unique(packed)) == n


def test_dropout_mask_statistics_and_special_cases():
    m0 = sp.dropout_mask(64, 128, 0.0, seed=7, offset=0)
    assert m0.all()
    for p in (0.1, 0.5):
        m = sp.dropout_mask(256, 512, p, seed=99, offset=8)
        n = m.size
        sd = math.sqrt(n * p * (1 - p))
        assert abs(m.sum() - n * (1 - p)) < 6 * sd
    a = sp.dropout_mask(16, 64, 0.3, seed=1, offset=0)
    b = sp.dropout_mask(16, 64, 0.3, seed=2, offset=0)
    assert (a != b).any()
    # the offset is an element counter: rows 1.. of one call are rows 0.. of a call offset by h
    big = sp.dropout_mask(5, 24, 0.4, seed=3, offset=16)
    shifted = sp.dropout_mask(4, 24, 0.4, seed=3, offset=16 + 24)
    assert np.array_equal(big[1:], shifted)
    assert sp.dropout_keep_threshold(0.0) == 1 << 32
    assert sp.dropout_keep_threshold(0.5) == 1 << 31


def test_bias_dropout_add_forward_and_backward():
    rng = _rng(6)
    Y, R, dO = rng.standard_normal((6, 40)), rng.standard_normal((6, 40)), rng.standard_normal((6, 40))
    b = rng.standard_normal(40)
    out0, m0 = sp.bias_dropout_add_fwd(Y, b, R, 0.0, 5, 0)
    np.testing.assert_array_equal(out0, R + (Y + b))
    p = 0.25
    out, m = sp.bias_dropout_add_fwd(Y, b, R, p, 5, 0)
    kept = (out - R)[m]
    np.testing.assert_allclose(kept, (Y + b)[m] / 0.75, rtol=0, atol=1e-14)   # out - R cancels
    assert np.all((out - R)[~m] == 0.0)
    dY, db, dR = sp.bias_dropout_add_bwd(dO, p, 5, 0)
    # the map Y -> out is linear with derivative mask / (1 - p)
    eps = 1e-3
    num = np.zeros_like(Y)
    for idx in np.ndindex(*Y.shape):
        Yp, Ym = Y.copy(), Y.copy()
        Yp[idx] += eps
        Ym[idx] -= eps
        num[idx] = (np.sum(dO * sp.bias_dropout_add_fwd(Yp, b, R, p, 5, 0)[0]) -
                    np.sum(dO * sp.bias_dropout_add_fwd(Ym, b, R, p, 5, 0)[0])) / (2 * eps)
    np.testing.assert_allclose(dY, num, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(db, num.sum(axis=0), rtol=1e-9, atol=1e-9)
    np.testing.assert_array_equal(dR, dO)


# ---------------------------------------------------------------- planted mistakes

def _pins_pass():
    try:
        test_rows_are_normalised()
        test_layernorm_bruteforce()
        test_layernorm_finite_differences()
        test_philox_known_answers()
        test_bias_dropout_add_forward_and_backward()
    except AssertionError:
        return False
    return True


def test_pins_pass_unplanted():
    assert _pins_pass()


def test_planted_unbiased_variance_is_caught(monkeypatch):
    def wrong(X, gamma, beta=None, eps=1e-5):
        X, g = np.asarray(X, float), np.asarray(gamma, float)
        mean = X.mean(axis=1)
        var = X.var(axis=1, ddof=1) if X.shape[1] > 1 else np.zeros(X.shape[0])
        rstd = 1.0 / np.sqrt(var + eps)
        Y = (X - mean[:, None]) * rstd[:, None] * g
        return (Y + np.asarray(beta, float) if beta is not None else Y), mean, rstd
    monkeypatch.setattr(sp, "layernorm_fwd", wrong)
    assert not _pins_pass()


def test_planted_philox_multiplier_swap_is_caught(monkeypatch):
    monkeypatch.setattr(sp, "PHILOX_M0", sp.PHILOX_M1)
    orig = sp.philox4x32_10

    def swapped(counter, key):
        c = np.array(counter, dtype=np.uint64) & sp._MASK32
        k = np.array(key, dtype=np.uint64) & sp._MASK32
        c0, c1, c2, c3 = (c[..., i] for i in range(4))
        k0, k1 = k[..., 0] + np.zeros_like(c0), k[..., 1] + np.zeros_like(c0)
        for r in range(10):
            if r > 0:
                k0 = (k0 + np.uint64(sp.PHILOX_W0)) & sp._MASK32
                k1 = (k1 + np.uint64(sp.PHILOX_W1)) & sp._MASK32
            p0, p1 = np.uint64(0xCD9E8D57) * c0, np.uint64(0xD2511F53) * c2
            c0, c1, c2, c3 = (p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & sp._MASK32, (p0 >> np.uint64(32)) ^ c3 ^ k1, \
                p0 & sp._MASK32
        return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)
    monkeypatch.setattr(sp, "philox4x32_10", swapped)
    assert not _pins_pass()
    monkeypatch.setattr(sp, "philox4x32_10", orig)


def test_planted_dropout_scale_and_ln_grad_mistakes_are_caught(monkeypatch):
    orig_fwd, orig_bwd = sp.bias_dropout_add_fwd, sp.layernorm_bwd

    def unscaled(Y, b, residual, p, seed, offset):
        Y, R = np.asarray(Y, float), np.asarray(residual, float)
        m = sp.dropout_mask(*Y.shape, p, seed, offset)
        return R + np.where(m, Y + (b if b is not None else 0.0), 0.0), m

    def no_xhat_term(X, gamma, dY, eps=1e-5):
        X, g, dY = (np.asarray(a, float) for a in (X, gamma, dY))
        _, mean, rstd = sp.layernorm_fwd(X, g, None, eps)
        xhat = (X - mean[:, None]) * rstd[:, None]
        gy = dY * g
        return rstd[:, None] * (gy - gy.mean(axis=1, keepdims=True)), (dY * xhat).sum(0), dY.sum(0)

    monkeypatch.setattr(sp, "bias_dropout_add_fwd", unscaled)
    assert not _pins_pass()
    monkeypatch.setattr(sp, "bias_dropout_add_fwd", orig_fwd)
    monkeypatch.setattr(sp, "layernorm_bwd", no_xhat_term)
    assert not _pins_pass()
    monkeypatch.setattr(sp, "layernorm_bwd", orig_bwd)
    assert _pins_pass()
