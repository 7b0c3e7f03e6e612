"""The C ABI: the library loads on a host without a GPU, exports every symbol
include/*.h declares, and rejects invalid arguments before touching the GPU.

Only validation paths are exercised here: each call below fails a check that
runs before any HIP call, so no pointer is dereferenced and nothing is
launched (the pointers are arbitrary aligned integers)."""
import ctypes
import glob
import os
import re

import pytest

from tensor_transformer_mlp_shard_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.LIB_PATH):
        import __graft_entry__  # builds the library in-tree
        __graft_entry__.build()
    return _native.lib()


def _declared():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(tp_\w+)\s*\(", text))
    return names


def test_header_declares_the_boundary():
    d = _declared()
    for n in ("tp_column_linear", "tp_row_linear", "tp_mlp_shard_fwd", "tp_mlp_shard_bwd",
              "tp_column_linear_bwd", "tp_row_linear_bwd", "tp_workspace_size", "tp_status_string"):
        assert n in d


def test_every_declared_symbol_is_exported(lib):
    d = _declared()
    assert d
    for name in d:
        assert hasattr(lib, name), name
        assert name in _native.PROTOTYPES, name


def test_status_strings(lib):
    for code in _native.STATUS:
        s = lib.tp_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.tp_status_string(12345).decode() == "unknown status"


P = ctypes.c_void_p
A0, A1, A2, A3, A4, A5, A6 = (P(0x10000 * (i + 1)) for i in range(7))   # 16-byte aligned, disjoint-ish
S = P(0)


def test_column_linear_validation(lib):
    f = lib.tp_column_linear
    ok = dict(T=128, K=256, N=1024, tp=2)
    # null pointers
    assert f(None, A1, None, A2, None, 128, 256, 1024, 2, 0, 0, S) == -1
    # non-positive dims
    assert f(A0, A1, None, A2, None, 0, 256, 1024, 2, 0, 0, S) == -2
    assert f(A0, A1, None, A2, None, 128, -8, 1024, 2, 0, 0, S) == -2
    assert f(A0, A1, None, A2, None, 1 << 31, 256, 1024, 2, 0, 0, S) == -2
    assert f(A0, A1, None, A2, None, 128, 1 << 22, 1024, 2, 0, 0, S) == -2     # feature dim > 2^21
    # TP divisibility
    assert f(A0, A1, None, A2, None, 128, 256, 1000, 3, 0, 0, S) == -3
    assert f(A0, A1, None, A2, None, 128, 256, 1024, 0, 0, 0, S) == -3
    # feature alignment: K not a multiple of 8, shard width not a multiple of 8
    assert f(A0, A1, None, A2, None, 128, 250, 1024, 2, 0, 0, S) == -4
    assert f(A0, A1, None, A2, None, 128, 256, 1028, 2, 0, 0, S) == -4
    # misaligned pointer
    assert f(P(0x10008), A1, None, A2, None, 128, 256, 1024, 2, 0, 0, S) == -4
    # dtype / activation codes
    assert f(A0, A1, None, A2, None, 128, 256, 1024, 2, 0, 7, S) == -5
    assert f(A0, A1, None, A2, None, 128, 256, 1024, 2, 5, 0, S) == -5
    # Z given without activation
    assert f(A0, A1, None, A2, A3, 128, 256, 1024, 2, 0, 0, S) == -9
    # output aliasing an input (Y_i == X)
    assert f(A0, A1, None, A0, None, 128, 256, 1024, 2, 0, 0, S) == -6
    # Z overlapping Y
    assert f(A0, A1, None, A2, P(A2.value + 64), 128, 256, 1024, 2, 1, 0, S) == -6


def test_row_linear_validation(lib):
    f = lib.tp_row_linear
    assert f(A0, None, None, A2, 128, 1024, 256, 2, 0, S) == -1
    assert f(A0, A1, None, A2, 128, 1024, 256, 3, 0, S) == -3
    assert f(A0, A1, None, A2, 128, 1032, 256, 2, 0, S) == -4    # K/p = 516 not a multiple of 8
    assert f(A0, A1, None, A1, 128, 1024, 256, 2, 0, S) == -6


def test_mlp_fwd_validation(lib):
    f = lib.tp_mlp_shard_fwd
    assert f(A0, A1, None, A2, None, None, A4, 128, 256, 1024, 2, 0, S) == -1     # H missing
    assert f(A0, A1, None, A2, None, A3, A4, 128, 256, 1024, 3, 0, S) == -3
    assert f(A0, A1, None, A2, None, A3, A4, 128, 260, 1024, 2, 0, S) == -4
    assert f(A0, A1, None, A2, A3, A3, A4, 128, 256, 1024, 2, 0, S) == -6          # Z == H
    assert f(A0, A1, None, A2, None, A3, A4, 128, 256, 1024, 2, 3, S) == -5          # no dtype 3


def test_mlp_bwd_validation(lib):
    f = lib.tp_mlp_shard_bwd
    need = lib.tp_workspace_size(_native.TP_OP_MLP_SHARD_BWD, 128, 256, 1024, 2, 0)
    assert need > 128 * 512 * 2
    base = [A0, A1, A2, A3, A4, A5, A6, P(0x100000), None, P(0x200000), None]
    ws = P(0x1000000)
    # workspace missing / too small
    assert f(*base, None, 0, 0, 128, 256, 1024, 2, 0, S) == -7
    assert f(*base, ws, need - 1, 0, 128, 256, 1024, 2, 0, S) == -7
    # bad accumulate flag
    assert f(*base, ws, need, 2, 128, 256, 1024, 2, 0, S) == -9
    # dA_i aliasing dB_i
    bad = list(base)
    bad[9] = bad[7]
    assert f(*bad, ws, need, 0, 128, 256, 1024, 2, 0, S) == -6


def test_linear_bwd_validation(lib):
    need = lib.tp_workspace_size(_native.TP_OP_ROW_LINEAR_BWD, 64, 512, 256, 2, 0)
    assert need >= 256 * 4
    f = lib.tp_row_linear_bwd
    assert f(A0, A1, A2, A3, A4, A5, None, 0, 0, 64, 512, 256, 2, 0, S) == -7   # db wanted, no workspace
    assert f(A0, A1, A2, A3, A4, A5, A6, need - 4, 0, 64, 512, 256, 2, 0, S) == -7
    g = lib.tp_column_linear_bwd
    assert g(A0, A1, A2, A0, A4, None, None, 0, 0, 64, 256, 512, 2, 0, S) == -6  # dX == X


def test_workspace_size(lib):
    ws = lib.tp_workspace_size
    assert ws(99, 128, 256, 1024, 2, 0) == 0
    assert ws(_native.TP_OP_MLP_SHARD_BWD, 0, 256, 1024, 2, 0) == 0
    assert ws(_native.TP_OP_MLP_SHARD_BWD, 128, 256, 1000, 3, 0) == 0
    a = ws(_native.TP_OP_MLP_SHARD_BWD, 2048, 12288, 49152, 8, 0)
    assert a >= 2048 * 6144 * 2
    assert ws(_native.TP_OP_MLP_SHARD_BWD, 2048, 12288, 49152, 8, 1) > a   # fp32 dZ
    assert ws(_native.TP_OP_BIAS_GRAD, 4096, 1024, 0, 1, 0) >= 1024 * 4
    assert ws(_native.TP_OP_COLUMN_LINEAR_BWD, 8192, 12288, 36864, 8, 0) >= 4608 * 4


def test_probe_validation(lib):
    # every call fails its argument checks before any HIP call
    assert lib.tp_mfma_probe(0, 10, A0, A1, S) == -9
    assert lib.tp_mfma_probe(65537, 10, A0, A1, S) == -9
    assert lib.tp_mfma_probe(4, 0, A0, A1, S) == -9
    assert lib.tp_mfma_probe(4, (1 << 24) + 1, A0, A1, S) == -9
    assert lib.tp_mfma_probe(4, 10, None, A1, S) == -1
    assert lib.tp_mfma_probe(4, 10, A0, None, S) == -1
    assert lib.tp_mfma_probe(4, 10, A0, P(0x10004), S) == -4
    assert lib.tp_wall_clock_rate_khz(None) == -1


def test_attention_fwd_validation(lib):
    f = lib.tp_attention_fwd
    A0, A1, A2 = P(0x1000000), P(0x2000000), P(0x3000000)   # disjoint at these sizes
    # (QKV, O, lse, T, seq, heads, head_dim, tp, causal, dtype, stream); 2 local heads of 64 -> QKV 384 wide
    assert f(A0, A1, A2, 256, 128, 4, 64, 2, 1, 1, S) == -5          # fp32: MFMA kernels are bf16 only
    assert f(A0, A1, A2, 256, 128, 4, 64, 2, 1, 7, S) == -5
    assert f(A0, A1, A2, 256, 128, 4, 64, 2, 1, 2, S) == -5          # fp16: not for attention
    assert f(A0, A1, A2, 256, 128, 4, 96, 2, 1, 0, S) == -2          # head_dim not 64/128
    assert f(A0, A1, A2, 250, 128, 4, 64, 2, 1, 0, S) == -2          # T not whole sequences
    assert f(A0, A1, A2, 0, 128, 4, 64, 2, 1, 0, S) == -2
    assert f(A0, A1, A2, 256, 0, 4, 64, 2, 1, 0, S) == -2
    assert f(A0, A1, A2, 256, 128, 4, 64, 3, 1, 0, S) == -3          # heads % tp
    assert f(A0, A1, A2, 256, 128, 4, 64, 0, 1, 0, S) == -3
    assert f(A0, A1, A2, 256, 128, 4, 64, 2, 2, 0, S) == -9          # causal flag
    assert f(None, A1, A2, 256, 128, 4, 64, 2, 1, 0, S) == -1
    assert f(A0, None, A2, 256, 128, 4, 64, 2, 1, 0, S) == -1
    assert f(P(0x10008), A1, A2, 256, 128, 4, 64, 2, 1, 0, S) == -4
    assert f(A0, A0, A2, 256, 128, 4, 64, 2, 1, 0, S) == -6          # O aliases QKV
    assert f(A0, A1, P(A1.value + 256), 256, 128, 4, 64, 2, 1, 0, S) == -6   # lse inside O
    assert f(A0, A1, A2, 1 << 20, 1 << 20, 3 * 4096, 128, 1, 1, 0, S) == -2  # QKV wider than 2^21


def test_attention_bwd_validation(lib):
    f = lib.tp_attention_bwd
    QKV, O, L, G, DQ, WS = (P(0x1000000 * (i + 1)) for i in range(6))
    need = lib.tp_workspace_size(_native.TP_OP_ATTENTION_BWD, 256, 4, 64, 2, 0)
    assert need >= 2 * 256 * 4
    assert lib.tp_workspace_size(_native.TP_OP_ATTENTION_BWD, 256, 4, 64, 2, 1) == 0      # fp32
    assert lib.tp_workspace_size(_native.TP_OP_ATTENTION_BWD, 256, 4, 96, 2, 0) == 0      # head_dim
    assert lib.tp_workspace_size(_native.TP_OP_ATTENTION_BWD, 256, 5, 64, 2, 0) == 0      # heads % tp
    args = (256, 128, 4, 64, 2, 1, 0, S)
    assert f(QKV, O, L, G, DQ, WS, need - 1, *args) == -7
    assert f(QKV, O, L, G, DQ, None, need, *args) == -7
    assert f(QKV, O, None, G, DQ, WS, need, *args) == -1                                  # lse required
    assert f(QKV, O, L, None, DQ, WS, need, *args) == -1
    assert f(QKV, O, L, G, QKV, WS, need, *args) == -6                                    # dQKV aliases QKV
    assert f(QKV, O, L, G, DQ, P(DQ.value + 4096), need, *args) == -6                     # workspace inside dQKV
    assert f(QKV, O, L, G, DQ, WS, need, 256, 128, 4, 64, 2, 1, 1, S) == -5
    assert f(QKV, O, L, G, DQ, WS, need, 256, 100, 4, 64, 2, 1, 0, S) == -2


def test_mlp_bwd_recompute_validation(lib):
    f = lib.tp_mlp_shard_bwd_recompute
    need = lib.tp_workspace_size(_native.TP_OP_MLP_SHARD_BWD_RECOMPUTE, 128, 256, 1024, 2, 0)
    assert need >= 3 * 128 * 512 * 2 > lib.tp_workspace_size(_native.TP_OP_MLP_SHARD_BWD, 128, 256, 1024, 2, 0)
    X, Ai, b1, Bi, Z, dY, dX, dA, db1, dB, db2, WS = (P(0x1000000 * (i + 1)) for i in range(12))
    args = (0, 128, 256, 1024, 2, 0, S)
    assert f(X, Ai, b1, Bi, Z, dY, dX, dA, db1, dB, db2, WS, need - 1, *args) == -7
    assert f(None, Ai, b1, Bi, Z, dY, dX, dA, db1, dB, db2, WS, need, *args) == -1
    assert f(X, Ai, b1, Bi, Z, dY, Z, dA, db1, dB, db2, WS, need, *args) == -6       # dX aliases Z
    assert f(X, Ai, b1, Bi, None, dY, dX, dA, db1, dB, db2, P(dA.value + 64), need, *args) == -6
    assert f(X, Ai, b1, Bi, Z, dY, dX, dA, db1, dB, db2, WS, need, 2, 128, 256, 1024, 2, 0, S) == -9
    assert f(X, Ai, b1, Bi, Z, dY, dX, dA, db1, dB, db2, WS, need, 0, 128, 256, 1024, 3, 0, S) == -3


def test_sp_edge_validation(lib):
    X, G, B, Y, M, R, DY, DX, DG, DB, WS = (P(0x1000000 * (i + 1)) for i in range(11))
    f = lib.tp_layernorm_fwd
    assert f(None, G, B, Y, M, R, 64, 1024, 1e-5, 0, S) == -1
    assert f(X, G, B, Y, M, None, 64, 1024, 1e-5, 0, S) == -9        # mean without rstd
    assert f(X, G, B, Y, M, R, 64, 1024, -1.0, 0, S) == -9            # eps < 0
    assert f(X, G, B, Y, M, R, 64, 1020, 1e-5, 0, S) == -4            # h not a multiple of 8
    assert f(X, G, B, Y, M, R, 0, 1024, 1e-5, 0, S) == -2
    assert f(X, G, B, X, M, R, 64, 1024, 1e-5, 0, S) == -6            # in place is rejected
    assert f(X, G, B, Y, M, R, 64, 1024, 1e-5, 3, S) == -5
    g = lib.tp_layernorm_bwd
    need = lib.tp_workspace_size(_native.TP_OP_LAYERNORM_BWD, 64, 1024, 0, 1, 0)
    assert need >= 2 * 8 * 1024 * 4
    assert g(X, G, M, R, DY, DX, DG, DB, WS, need - 1, 0, 64, 1024, 0, S) == -7
    assert g(X, G, M, R, DY, DX, None, DB, WS, need, 0, 64, 1024, 0, S) == -1
    assert g(X, G, M, R, DY, DX, DG, DB, WS, need, 2, 64, 1024, 0, S) == -9
    assert g(X, G, M, R, DY, DY, DG, DB, WS, need, 0, 64, 1024, 0, S) == -6
    d = lib.tp_bias_dropout_add_fwd
    assert d(Y, B, X, DX, 64, 1024, 1.0, 1, 0, 0, S) == -9             # p = 1
    assert d(Y, B, X, DX, 64, 1024, -0.1, 1, 0, 0, S) == -9
    assert d(Y, B, X, DX, 64, 1024, 0.1, 1, 4, 0, S) == -9             # offset not a multiple of 8
    assert d(Y, B, X, X, 64, 1024, 0.1, 1, 0, 0, S) == -6
    assert d(None, B, X, DX, 64, 1024, 0.1, 1, 0, 0, S) == -1
    e = lib.tp_bias_dropout_add_bwd
    need2 = lib.tp_workspace_size(_native.TP_OP_BIAS_DROPOUT_ADD_BWD, 64, 1024, 0, 1, 0)
    assert need2 > 0
    assert e(DY, DX, DG, None, 0, 0, 64, 1024, 0.1, 1, 0, 0, S) == -7  # db wanted, no workspace
    assert e(DY, DY, None, None, 0, 0, 64, 1024, 0.1, 1, 0, 0, S) == -6
    assert e(DY, DX, None, None, 0, 0, 64, 1024, 0.1, 1, 12, 0, S) == -9


def test_unscale_check_validation(lib):
    f = lib.tp_unscale_check_finite
    G, F = P(0x1000000), P(0x2000000)
    assert f(None, 16, ctypes.c_float(0.5), F, S) == -1
    assert f(G, 16, ctypes.c_float(0.5), None, S) == -1
    assert f(G, 0, ctypes.c_float(0.5), F, S) == -2
    assert f(G, 16, ctypes.c_float(0.0), F, S) == -9
    assert f(G, 16, ctypes.c_float(float("inf")), F, S) == -9
    assert f(G, 16, ctypes.c_float(float("nan")), F, S) == -9
    assert f(P(0x1000004), 16, ctypes.c_float(0.5), F, S) == -4
    assert f(G, 16, ctypes.c_float(0.5), P(0x1000008), S) == -6        # flag inside the buffer


# Addresses far apart, so that no overlap check fires before the size checks.
FAR = [P((i + 1) << 40) for i in range(12)]


def test_launch_size_limits(lib):
    """Sizes inside the dimension and element limits whose launch would pass
    the 32-bit dispatch size (2^32 - 1 work-items) are rejected with
    TP_ERR_DIM before anything is enqueued."""
    X, W, B, Y, Z, R = FAR[:6]
    # elementwise passes: one work-item per 8 elements -> T*N = 2^36 needs 2^33
    assert lib.tp_bias_gelu(X, B, Y, 1 << 20, 1 << 16, 0, S) == -2
    assert lib.tp_bias_dropout_add_fwd(X, B, R, Y, 1 << 20, 1 << 16, 0.1, 1, 0, 0, S) == -2
    assert lib.tp_bias_dropout_add_bwd(X, Y, None, None, 0, 0, 1 << 20, 1 << 16, 0.1, 1, 0, 0, S) == -2
    # LayerNorm forward: one 256-wide workgroup per row -> 2^24 rows need 2^32
    assert lib.tp_layernorm_fwd(X, W, B, Y, Z, R, 1 << 24, 8, 1e-5, 0, S) == -2
    # attention: one 256-wide workgroup per 128 queries of a (sequence, head):
    # 2^18 sequences of 128 tokens x 1024 local heads of 64 -> 2^36 work-items
    assert lib.tp_attention_fwd(X, Y, Z, 1 << 25, 128, 1024, 64, 1, 1, 0, S) == -2
    # fp32 GEMM: 64 x 64 tiles of 256 work-items; 2^30 tokens x 64 outputs -> 2^32
    assert lib.tp_column_linear(X, W, None, Y, None, 1 << 30, 8, 64, 1, 0, 1, S) == -2
    assert lib.tp_row_linear(X, W, None, Y, 1 << 30, 8, 64, 1, 1, S) == -2
    assert lib.tp_mlp_shard_fwd(X, W, None, B, None, Z, Y, 1 << 30, 8, 64, 1, 1, S) == -2
    ws = FAR[11]
    need = lib.tp_workspace_size(_native.TP_OP_COLUMN_LINEAR_BWD, 1 << 30, 8, 64, 1, 1)
    assert need > 0
    assert lib.tp_column_linear_bwd(X, W, B, Y, Z, None, ws, need, 0, 1 << 30, 64, 8, 1, 1, S) == -2
    assert lib.tp_row_linear_bwd(X, W, B, Y, Z, None, ws, need, 0, 1 << 30, 8, 64, 1, 1, S) == -2
    assert lib.tp_mlp_shard_bwd(X, W, B, Z, R, FAR[6], FAR[7], FAR[8], None, FAR[9], None, ws, 1 << 62, 0,
                                1 << 30, 8, 64, 1, 1, S) == -2


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """tp_mlp_shard_bwd_noalloc checks the problem's scratch against its static
    array before any HIP call (1.3B TP=1 in fp32 needs 130 MiB of 96)."""
    cap = lib.tp_noalloc_scratch_bytes()
    assert cap == 96 << 20
    need = lib.tp_workspace_size(_native.TP_OP_MLP_SHARD_BWD, 4096, 2048, 8192, 1, 1)
    assert need > cap
    X, A, B, Z, H, dY, dX, dA, db1, dB = FAR[:10]
    assert lib.tp_mlp_shard_bwd_noalloc(X, A, B, Z, H, dY, dX, dA, db1, dB, None, 0, 4096, 2048, 8192, 1, 1, S) == -10
    # the ordinary checks come first
    assert lib.tp_mlp_shard_bwd_noalloc(X, A, B, Z, H, dY, dX, dA, db1, dB, None, 2, 4096, 2048, 8192, 1, 1, S) == -9
    assert lib.tp_mlp_shard_bwd_noalloc(X, A, B, Z, H, dY, X, dA, db1, dB, None, 0, 4096, 2048, 8192, 1, 1, S) == -6


def test_workspace_holds_the_k_split_partial(lib):
    """A 16-bit weight gradient whose tiles fill at most half of the CUs splits
    its contraction in two; the workspace then holds its M x N fp32 partial
    besides the bias-gradient rows.  Large weight gradients and the fp32 path do
    not split."""
    bf16, fp32 = 0, 1
    # column shard dW [1024 x 1024], contraction 4096: 64 tiles of 128 x 128
    need = lib.tp_workspace_size(_native.TP_OP_COLUMN_LINEAR_BWD, 4096, 1024, 2048, 2, bf16)
    assert need >= 1024 * 1024 * 4
    # row shard dW [512 x 2048], contraction 2080 (65 steps of 32)
    assert lib.tp_workspace_size(_native.TP_OP_ROW_LINEAR_BWD, 2080, 1024, 2048, 2, bf16) >= 512 * 2048 * 4
    # MLP at GPT h=1024 TP=2: dZ [4096 x 2048] bf16, then room for a [2048 x 1024] partial
    assert lib.tp_workspace_size(_native.TP_OP_MLP_SHARD_BWD, 4096, 1024, 4096, 2, bf16) >= \
        4096 * 2048 * 2 + 2048 * 1024 * 4
    # 175B QKV weight gradient [12288 x 4608]: 768 tiles, no split
    assert lib.tp_workspace_size(_native.TP_OP_COLUMN_LINEAR_BWD, 8192, 12288, 36864, 8, bf16) < 12288 * 4608
    # a contraction under 64 steps of 32 does not split
    assert lib.tp_workspace_size(_native.TP_OP_COLUMN_LINEAR_BWD, 2016, 1024, 2048, 2, bf16) < 1024 * 1024
    assert lib.tp_workspace_size(_native.TP_OP_COLUMN_LINEAR_BWD, 4096, 1024, 2048, 2, fp32) < 1024 * 1024 * 4
