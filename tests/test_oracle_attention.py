"""Pins of the fp64 core-attention oracle (oracle/attention.py) against facts
that do not come from the oracle itself: closed forms, an independent
brute-force evaluation, invariances of softmax attention, finite differences
for the backward, the tensor-parallel head split, and planted mistakes that
one of these must catch.  CPU only."""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as att


def _qkv(rng, T, Hl, d, sigma=1.0):
    return rng.standard_normal((T, 3 * Hl * d)) * sigma


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("S,d", [(1, 4), (7, 8), (33, 16)])
def test_zero_queries_give_running_mean_of_values(S, d):
    """q = 0 makes every allowed score 0: causal attention then averages the
    values of keys 0..t, and lse_t = log(t + 1)."""
    rng = np.random.default_rng(1)
    Hl = 2
    QKV = _qkv(rng, 2 * S, Hl, d)
    QKV[:, : Hl * d] = 0.0
    O, lse = oracle.core_attention_fwd(QKV, S, Hl, d, causal=True)
    V = QKV[:, 2 * Hl * d:]
    for b0 in (0, S):
        Vs = V[b0: b0 + S]
        running = np.cumsum(Vs, axis=0) / np.arange(1, S + 1)[:, None]
        np.testing.assert_allclose(O[b0: b0 + S], running, rtol=0, atol=1e-13)
        for h in range(Hl):
            np.testing.assert_allclose(lse[h, b0: b0 + S], np.log(np.arange(1, S + 1)), rtol=0, atol=1e-13)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(2)
    QKV = _qkv(rng, 5, 3, 8)
    O, lse = oracle.core_attention_fwd(QKV, 1, 3, 8, causal=False)
    np.testing.assert_array_equal(O, QKV[:, 2 * 24:])
    q, k = QKV[:, :24].reshape(5, 3, 8), QKV[:, 24:48].reshape(5, 3, 8)
    np.testing.assert_allclose(lse.T, np.sum(q * k, axis=2) / math.sqrt(8), rtol=1e-14, atol=1e-14)


def test_hard_attention_selects_the_matching_key():
    """Query t aligned with key pi(t) <= t and orthogonal to every other key:
    the softmax is one-hot to within exp(-800), so O_t = V_pi(t)."""
    S, d = 8, 8
    rng = np.random.default_rng(3)
    pi = [int(rng.integers(0, t + 1)) for t in range(S)]
    K = np.eye(d)[:S] * 10.0
    Q = np.stack([np.eye(d)[pi[t]] * 80.0 * math.sqrt(d) for t in range(S)])
    V = rng.standard_normal((S, d))
    O, lse, P = oracle.attention_head_fwd(Q, K, V, causal=True)
    np.testing.assert_allclose(O, V[pi], rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.diag(P[:, pi]), 1.0, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- brute force

def _brute(QKV, S, Hl, d, causal):
    """Independent evaluation with Python floats: explicit loops, softmax
    without the max shift, causal mask as a loop bound."""
    T = len(QKV)
    O = [[0.0] * (Hl * d) for _ in range(T)]
    lse = [[0.0] * T for _ in range(Hl)]
    for h in range(Hl):
        for b0 in range(0, T, S):
            for i in range(S):
                q = [QKV[b0 + i][h * d + c] for c in range(d)]
                last = i if causal else S - 1
                w = []
                for j in range(last + 1):
                    k = [QKV[b0 + j][Hl * d + h * d + c] for c in range(d)]
                    w.append(math.exp(sum(q[c] * k[c] for c in range(d)) / math.sqrt(d)))
                tot = sum(w)
                lse[h][b0 + i] = math.log(tot)
                for c in range(d):
                    O[b0 + i][h * d + c] = sum(w[j] * QKV[b0 + j][2 * Hl * d + h * d + c] for j in range(last + 1)) / tot
    return np.array(O), np.array(lse)


@pytest.mark.parametrize("S,B,Hl,d,causal", [(1, 3, 2, 2, True), (3, 2, 2, 4, True), (5, 2, 3, 3, True),
                                             (4, 2, 2, 5, False), (6, 1, 1, 8, True)])
def test_bruteforce_tiny(S, B, Hl, d, causal):
    rng = np.random.default_rng(10 + S + d)
    QKV = _qkv(rng, S * B, Hl, d)
    O, lse = oracle.core_attention_fwd(QKV, S, Hl, d, causal)
    Ob, lseb = _brute(QKV.tolist(), S, Hl, d, causal)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- invariances

def test_key_shift_leaves_output_and_shifts_lse():
    """Adding one vector w to every key adds q_t.w / sqrt(d) to every score of
    row t: O is unchanged and lse_t moves by that amount."""
    rng = np.random.default_rng(4)
    S, d = 16, 8
    q, k, v = (rng.standard_normal((S, d)) for _ in range(3))
    w = rng.standard_normal(d)
    O0, lse0, _ = oracle.attention_head_fwd(q, k, v)
    O1, lse1, _ = oracle.attention_head_fwd(q, k + w, v)
    np.testing.assert_allclose(O1, O0, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse1 - lse0, q @ w / math.sqrt(d), rtol=1e-11, atol=1e-12)


def test_noncausal_key_permutation_invariance():
    rng = np.random.default_rng(5)
    S, d = 12, 8
    q, k, v = (rng.standard_normal((S, d)) for _ in range(3))
    perm = rng.permutation(S)
    O0, lse0, _ = oracle.attention_head_fwd(q, k, v, causal=False)
    O1, lse1, _ = oracle.attention_head_fwd(q, k[perm], v[perm], causal=False)
    np.testing.assert_allclose(O1, O0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0, rtol=1e-13, atol=1e-13)


def test_rows_of_p_are_distributions_over_allowed_keys():
    rng = np.random.default_rng(6)
    S, d = 20, 8
    q, k, v = (rng.standard_normal((S, d)) * 2 for _ in range(3))
    _, _, P = oracle.attention_head_fwd(q, k, v, causal=True)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(P[np.triu_indices(S, 1)] == 0.0)
    assert np.all(P[np.tril_indices(S)] > 0.0)


@pytest.mark.parametrize("p", [2, 4])
def test_head_split_across_ranks(p):
    """Column-parallel QKV gives each rank whole heads: the full layer's
    attention output is the concatenation of the ranks' outputs."""
    rng = np.random.default_rng(7)
    T, S, H, d = 12, 6, 8, 4
    Qf, Kf, Vf = (rng.standard_normal((T, H * d)) for _ in range(3))
    O_full, lse_full = oracle.core_attention_fwd(np.concatenate([Qf, Kf, Vf], 1), S, H, d)
    Hl = H // p
    parts, lses = [], []
    for r in range(p):
        cols = slice(r * Hl * d, (r + 1) * Hl * d)
        O_r, lse_r = oracle.core_attention_fwd(np.concatenate([Qf[:, cols], Kf[:, cols], Vf[:, cols]], 1), S, Hl, d)
        parts.append(O_r)
        lses.append(lse_r)
    np.testing.assert_array_equal(np.concatenate(parts, 1), O_full)
    np.testing.assert_array_equal(np.concatenate(lses, 0), lse_full)


def test_175b_shard_widths():
    """The 175B rank's QKV shard width 4608 is 3 x 12 heads x 128."""
    H, d, p = 12288 // 128, 128, 8
    assert 3 * (H // p) * d == 4608 == 36864 // 8


# ---------------------------------------------------------------- backward

def _fd_check(QKV, dO, S, Hl, d, causal, eps=1e-6):
    g = oracle.core_attention_bwd(QKV, dO, S, Hl, d, causal)
    num = np.zeros_like(QKV)
    for idx in np.ndindex(*QKV.shape):
        a, b = QKV.copy(), QKV.copy()
        a[idx] += eps
        b[idx] -= eps
        La = np.sum(dO * oracle.core_attention_fwd(a, S, Hl, d, causal)[0])
        Lb = np.sum(dO * oracle.core_attention_fwd(b, S, Hl, d, causal)[0])
        num[idx] = (La - Lb) / (2 * eps)
    return np.linalg.norm(g - num) / np.linalg.norm(num)


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences(causal):
    rng = np.random.default_rng(8)
    S, B, Hl, d = 4, 2, 2, 3
    QKV = _qkv(rng, S * B, Hl, d)
    dO = rng.standard_normal((S * B, Hl * d))
    assert _fd_check(QKV, dO, S, Hl, d, causal) < 1e-7


def test_backward_rowsum_identity():
    """rowsum(P * dP) = rowsum(dO * O): the two forms of the softmax Jacobian term."""
    rng = np.random.default_rng(9)
    S, d = 10, 6
    q, k, v, dO = (rng.standard_normal((S, d)) for _ in range(4))
    O, _, P = oracle.attention_head_fwd(q, k, v)
    dP = dO @ v.T
    np.testing.assert_allclose(np.sum(P * dP, 1), np.sum(dO * O, 1), rtol=1e-12, atol=1e-12)


def test_backward_with_stored_output():
    """The stored-output form of the backward (D from the given O) equals the
    default when O is the exact forward output, and with a perturbed O only
    dQ and dK move, by exactly ds = -P * delta(D) through K and Q."""
    rng = np.random.default_rng(10)
    S, B, Hl, d = 6, 2, 2, 4
    QKV = _qkv(rng, S * B, Hl, d)
    dO = rng.standard_normal((S * B, Hl * d))
    O, _ = oracle.core_attention_fwd(QKV, S, Hl, d, True)
    base = oracle.core_attention_bwd(QKV, dO, S, Hl, d, True)
    np.testing.assert_allclose(oracle.core_attention_bwd(QKV, dO, S, Hl, d, True, O=O), base, rtol=1e-12, atol=1e-12)
    Op = O + 1e-3 * rng.standard_normal(O.shape)
    got = oracle.core_attention_bwd(QKV, dO, S, Hl, d, True, O=Op)
    w = Hl * d
    np.testing.assert_array_equal(got[:, 2 * w:], base[:, 2 * w:])        # dV does not use D
    # one head of one sequence by hand: dQ moves by -(P * dD) K / sqrt(d)
    q, k = QKV[:S, :d], QKV[:S, w:w + d]
    _, _, P = oracle.attention_head_fwd(q, k, QKV[:S, 2 * w:2 * w + d], True)
    dD = np.sum(dO[:S, :d] * (Op[:S, :d] - O[:S, :d]), axis=1, keepdims=True)
    np.testing.assert_allclose(got[:S, :d] - base[:S, :d], -(P * dD) @ k / np.sqrt(d), rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def _pins_pass():
    try:
        test_zero_queries_give_running_mean_of_values(7, 8)
        test_bruteforce_tiny(5, 2, 3, 3, True)
        test_bruteforce_tiny(4, 2, 2, 5, False)
        test_finite_differences(True)
    except AssertionError:
        return False
    return True


def test_pins_pass_unplanted():
    assert _pins_pass()


def test_planted_mask_direction_is_caught(monkeypatch):
    def wrong(q, k, causal):
        S, d = q.shape
        s = (q @ k.T) / math.sqrt(d)
        if causal:
            i, j = np.arange(S)[:, None], np.arange(S)[None, :]
            s = np.where(j < i, -np.inf, s)
        return s
    monkeypatch.setattr(att, "_scores", wrong)
    assert not _pins_pass()


def test_planted_missing_scale_is_caught(monkeypatch):
    def wrong(q, k, causal):
        S, d = q.shape
        s = q @ k.T
        if causal:
            i, j = np.arange(S)[:, None], np.arange(S)[None, :]
            s = np.where(j > i, -np.inf, s)
        return s
    monkeypatch.setattr(att, "_scores", wrong)
    assert not _pins_pass()


def test_planted_head_layout_mistake_is_caught(monkeypatch):
    def wrong(QKV, heads_local, d):
        QKV = np.asarray(QKV, dtype=np.float64)
        T = QKV.shape[0]
        blocks = QKV.reshape(T, heads_local, 3, d)      # [head][q|k|v][d] instead of [q|k|v][head][d]
        return tuple(np.ascontiguousarray(blocks[:, :, i].transpose(1, 0, 2)) for i in range(3))
    monkeypatch.setattr(att, "split_qkv", wrong)
    assert not _pins_pass()


def test_planted_backward_mistakes_are_caught(monkeypatch):
    orig = att.attention_head_bwd

    def no_rowsum(q, k, v, dO, causal=True, o=None):
        q, k, v, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dO))
        d = q.shape[1]
        _, _, P = att.attention_head_fwd(q, k, v, causal)
        ds = P * (dO @ v.T)
        return (ds @ k) / math.sqrt(d), (ds.T @ q) / math.sqrt(d), P.T @ dO

    def untransposed_dv(q, k, v, dO, causal=True, o=None):
        dQ, dK, _ = orig(q, k, v, dO, causal, o)
        _, _, P = att.attention_head_fwd(q, k, v, causal)
        return dQ, dK, P @ np.asarray(dO, dtype=np.float64)

    for bad in (no_rowsum, untransposed_dv):
        monkeypatch.setattr(att, "attention_head_bwd", bad)
        assert not _pins_pass()
    monkeypatch.setattr(att, "attention_head_bwd", orig)
    assert _pins_pass()
