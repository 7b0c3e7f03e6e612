"""Every entry point's work captured in a HIP graph (through torch) and replayed:
nothing the library enqueues may break capture (no host synchronisation, no
allocation, no memset nodes), and a replay must write exactly what the eager
call writes.  Each case runs eagerly once for the reference, is captured once,
then replayed three times with an eager call and a synchronisation between the
replays and the graph's outputs cleared before each replay; every replay is
compared bitwise with the eager outputs.  Parity with the oracle is the other
GPU tests' business; this checks the replayed path against the eager one."""
import pytest
import torch

import tensor_transformer_mlp_shard_amd as tps
from tensor_transformer_mlp_shard_amd import _native, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(a).to(DEV) if not isinstance(a, torch.Tensor) else a.to(DEV)


def _replays_match(fn):
    """fn() enqueues the work and returns its output tensors (a list)."""
    ref = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the capture stream, as torch asks
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    for r in range(3):
        fn()                                  # eager work between the replays
        torch.cuda.synchronize()
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        bad = [i for i, (t, e) in enumerate(zip(outs, ref)) if not torch.equal(t, e)]
        print(f"  replay {r}: {'bitwise equal' if not bad else 'outputs ' + str(bad) + ' differ'}", flush=True)
        assert not bad


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_graph_mlp_fwd_bwd(dtype):
    T, h, F, p = 1000, 512, 4096, 2
    print(f"case MLP T={T} h={h} F={F} p={p} {dtype}", flush=True)
    d = synth.mlp_inputs(T, h, F, p, dtype, 0.05, seed=5101, full=False)
    X, A, b1, B, dY = (dev(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    ws = torch.empty((tps.workspace_size(_native.TP_OP_MLP_SHARD_BWD, T, h, F, p, X.dtype),), dtype=torch.uint8,
                     device=DEV)

    def run():
        Z, H, Y = tps.mlp_shard_fwd(X, A, b1, B, tp_size=p)
        g = tps.mlp_shard_bwd(X, A, B, Z, H, dY, tp_size=p, want_db2=True, workspace=ws)
        return [Z, H, Y] + [g[k] for k in ("dX", "dA", "dB", "db1", "db2")]

    _replays_match(run)


def test_graph_mlp_bwd_recompute_and_noalloc():
    T, h, F, p = 777, 256, 2048, 1
    print(f"case MLP recompute + allocation-free T={T} h={h} F={F}", flush=True)
    d = synth.mlp_inputs(T, h, F, p, "bf16", 0.05, seed=5103, full=False)
    X, A, b1, B, dY = (dev(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    Z, H, _ = tps.mlp_shard_fwd(X, A, b1, B, tp_size=p)
    ws = torch.empty((tps.workspace_size(_native.TP_OP_MLP_SHARD_BWD_RECOMPUTE, T, h, F, p, X.dtype),),
                     dtype=torch.uint8, device=DEV)
    f32 = torch.float32
    na = {"dX": torch.empty_like(X), "dA": torch.empty((h, F), dtype=f32, device=DEV),
          "dB": torch.empty((F, h), dtype=f32, device=DEV), "db1": torch.empty((F,), dtype=f32, device=DEV)}

    def run():
        kz = tps.mlp_shard_bwd(X, A, B, Z, None, dY, tp_size=p, recompute=True, workspace=ws)
        kn = tps.mlp_shard_bwd(X, A, B, None, None, dY, tp_size=p, recompute=True, b1_i=b1, workspace=ws)
        nz = tps.mlp_shard_bwd_noalloc(X, A, B, Z, H, dY, tp_size=p, out=na)
        return [kz[k] for k in ("dX", "dA", "dB", "db1")] + [kn[k] for k in ("dX", "dA", "dB", "db1")] + \
            [nz[k] for k in ("dX", "dA", "dB", "db1")]

    _replays_match(run)


def test_graph_linears_fwd_bwd():
    T, K, N, p = 1500, 1024, 3072, 2
    print(f"case linears T={T} K={K} N={N} p={p}", flush=True)
    g = synth.seeded(5107)
    X = dev(synth.randn(g, (T, K), 1.0, "bf16"))
    Wc = dev(synth.randn(g, (K, N // p), 0.03, "bf16"))
    bc = dev(synth.randn(g, (N // p,), 0.5, "bf16"))
    Xr = dev(synth.randn(g, (T, K // p), 1.0, "bf16"))
    Wr = dev(synth.randn(g, (K // p, N), 0.03, "bf16"))
    br = dev(synth.randn(g, (N,), 0.5, "bf16"))
    dYc = dev(synth.randn(g, (T, N // p), 1.0, "bf16"))
    dYr = dev(synth.randn(g, (T, N), 1.0, "bf16"))
    wsc = torch.empty((tps.workspace_size(_native.TP_OP_COLUMN_LINEAR_BWD, T, K, N, p, X.dtype),),
                      dtype=torch.uint8, device=DEV)
    wsr = torch.empty((tps.workspace_size(_native.TP_OP_ROW_LINEAR_BWD, T, K, N, p, X.dtype),),
                      dtype=torch.uint8, device=DEV)

    def run():
        Yc, Zc = tps.column_linear(X, Wc, bc, tp_size=p, act="gelu", save_z=True)
        Yr = tps.row_linear(Xr, Wr, br, tp_size=p)
        gc = tps.column_linear_bwd(X, Wc, dYc, tp_size=p, workspace=wsc)
        gr = tps.row_linear_bwd(Xr, Wr, dYr, tp_size=p, workspace=wsr)
        return [Yc, Zc, Yr] + [gc[k] for k in ("dX", "dW", "db")] + [gr[k] for k in ("dX", "dW", "db")]

    _replays_match(run)


def test_graph_attention_fwd_bwd():
    B, S, heads, d, p = 2, 320, 8, 128, 2
    T = B * S
    print(f"case attention B={B} S={S} heads={heads} d={d} p={p}", flush=True)
    x = synth.core_attn_inputs(T, heads // p, d, "bf16", 1.0, seed=5109)
    qkv, dO = dev(x["QKV"]), dev(x["dO"])
    kw = dict(seq=S, heads=heads, head_dim=d, tp_size=p, causal=True)
    ws = torch.empty((tps.workspace_size(_native.TP_OP_ATTENTION_BWD, T, heads, d, p, torch.bfloat16),),
                     dtype=torch.uint8, device=DEV)

    def run():
        O, lse = tps.attention_fwd(qkv, **kw)
        dqkv = tps.attention_bwd(qkv, O, lse, dO, workspace=ws, **kw)
        return [O, lse, dqkv]

    _replays_match(run)


def test_graph_sp_edge():
    rows, h = 700, 2048
    print(f"case SP edge rows={rows} h={h}", flush=True)
    x = synth.sp_edge_inputs(rows, h, "bf16", 0.1, seed=5113)
    X, gam, bet, dYl, Y, bias, R, dOut = (dev(x[k]) for k in ("X", "gamma", "beta", "dY_ln", "Y", "b", "residual",
                                                               "dOut"))
    wsl = torch.empty((tps.workspace_size(_native.TP_OP_LAYERNORM_BWD, rows, h, 0, 1, X.dtype),), dtype=torch.uint8,
                      device=DEV)
    wsd = torch.empty((tps.workspace_size(_native.TP_OP_BIAS_DROPOUT_ADD_BWD, rows, h, 0, 1, X.dtype),),
                      dtype=torch.uint8, device=DEV)

    def run():
        y, mean, rstd = tps.layernorm_fwd(X, gam, bet)
        gl = tps.layernorm_bwd(X, gam, mean, rstd, dYl, workspace=wsl)
        o = tps.bias_dropout_add_fwd(Y, bias, R, p=0.1, seed=1234, offset=8)
        dy, db = tps.bias_dropout_add_bwd(dOut, p=0.1, seed=1234, offset=8, workspace=wsd)
        return [y, mean, rstd, gl["dX"], gl["dgamma"], gl["dbeta"], o, dy, db]

    _replays_match(run)
