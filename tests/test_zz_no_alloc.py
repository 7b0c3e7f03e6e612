"""The allocation-free MLP backward (tp_mlp_shard_bwd_noalloc, scratch in the
library's static device array) against the entry point with a caller
workspace (tp_mlp_shard_bwd), through the C ABI: the two run the same
kernels, so their outputs must be bitwise equal.  Two calls in a row, the
second on a smaller, ragged problem (the array then holds the first call's
contents), in bf16 and fp16, plus the accumulate form; the smaller problem is
also checked against the fp64 oracle, and a problem larger than the array is
rejected."""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_shard_amd as tps
from tensor_transformer_mlp_shard_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("dX", "dA", "dB", "db1", "db2")


def _case(T, h, F, p, dt, seed):
    d = synth.mlp_inputs(T, h, F, p, dt, 0.02, seed=seed, full=False)
    x = {k: d[k].to(DEV) for k in ("X", "A", "b1", "B", "dY")}
    z, hh, _ = tps.mlp_shard_fwd(x["X"], x["A"], x["b1"], x["B"], tp_size=p)
    return d, x, z, hh


def _outs(T, h, f, dt):
    e = lambda shape, t: torch.full(shape, float("nan"), dtype=t, device=DEV)  # noqa: E731
    return {"dX": e((T, h), dt), "dA": e((h, f), torch.float32), "dB": e((f, h), torch.float32),
            "db1": e((f,), torch.float32), "db2": e((h,), torch.float32)}


def _run_pair(T, h, F, p, dt, seed, accumulate=False):
    f = F // p
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dt]
    d, x, z, hh = _case(T, h, F, p, dt, seed)
    ref = _outs(T, h, f, tdt)
    got = _outs(T, h, f, tdt)
    if accumulate:
        g = torch.Generator(device="cpu").manual_seed(seed + 1)
        for k in ("dA", "dB", "db1", "db2"):
            init = torch.randn(ref[k].shape, generator=g).to(DEV)
            ref[k].copy_(init)
            got[k].copy_(init)
    tps.mlp_shard_bwd(x["X"], x["A"], x["B"], z, hh, x["dY"], tp_size=p, want_db2=True, out=ref,
                      accumulate=accumulate)
    tps.mlp_shard_bwd_noalloc(x["X"], x["A"], x["B"], z, hh, x["dY"], tp_size=p, want_db2=True, out=got,
                              accumulate=accumulate)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(got[k], ref[k]), f"{k} differs from tp_mlp_shard_bwd ({dt}, T={T} h={h} F={F} p={p})"
    return d, got


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_noalloc_matches_workspace_entry_point_twice(dt):
    print(f"noalloc {dt}: GPT h=1024 TP=2 shard, then a ragged small one", flush=True)
    _run_pair(4096, 1024, 4096, 2, dt, 71)                       # 16 MiB of scratch
    d, got = _run_pair(300, 256, 1568, 4, dt, 72)               # smaller, ragged: T=300, f=392
    # the smaller call also against the oracle
    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    X, A, b1, B, dY = (f64(d[k]) for k in ("X", "A", "b1", "B", "dY"))
    r = oracle.mlp_shard_bwd(X, A, b1, B, dY)
    for k, ref in (("dX", r["dX"]), ("dA", r["dA"]), ("dB", r["dB"]), ("db1", r["db1"]),
                   ("db2", oracle.bias_grad(dY))):
        e = oracle.rel_fro(f64(got[k]), ref)
        print(f"  {k:4s} rel_fro={e:.3e}", flush=True)
        assert e <= 5e-3


def test_noalloc_accumulate_and_175b_shape():
    print("noalloc bf16: 175B TP=8 shard with accumulate", flush=True)
    _run_pair(2048, 12288, 49152, 8, "bf16", 73, accumulate=True)   # 26 MiB of scratch
    _run_pair(1, 64, 512, 2, "bf16", 74, accumulate=True)            # one token


def test_noalloc_rejects_problem_larger_than_scratch():
    # 1.3B TP=1 in fp32 needs 130 MiB of scratch (dZ in fp32), the array holds 96 MiB
    T, h, F = 4096, 2048, 8192
    need = tps.workspace_size(tps._native.TP_OP_MLP_SHARD_BWD, T, h, F, 1, torch.float32)
    assert need > tps.noalloc_scratch_bytes()
    x = torch.empty((T, h), device=DEV)
    a = torch.empty((h, F), device=DEV)
    b = torch.empty((F, h), device=DEV)
    z = torch.empty((T, F), device=DEV)
    hh = torch.empty((T, F), device=DEV)
    out = {"dX": torch.empty((T, h), device=DEV), "dA": torch.empty((h, F), device=DEV),
           "dB": torch.empty((F, h), device=DEV), "db1": torch.empty((F,), device=DEV)}
    with pytest.raises(RuntimeError, match="TP_ERR_SCRATCH"):
        tps.mlp_shard_bwd_noalloc(x, a, b, z, hh, x, tp_size=1, out=out)
