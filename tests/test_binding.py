"""The Python binding validates every tensor it hands to the C ABI -- caller-
supplied outputs included -- before any call into the library.

Runs on the CPU: the GPU-placement check is switched off and the library is
replaced by a stub that fails the test if anything reaches it, so only the
binding's own argument checks run."""
import pytest
import torch

import tensor_transformer_mlp_shard_amd as tps
from tensor_transformer_mlp_shard_amd import _native


class _NoLibrary:
    def __getattr__(self, name):
        if name == "tp_workspace_size":
            return lambda *a: 1024
        raise AssertionError(f"{name} reached the library although an argument was invalid")


@pytest.fixture(autouse=True)
def cpu_binding(monkeypatch):
    monkeypatch.setattr(tps, "_require_gpu", lambda name, t: None)
    monkeypatch.setattr(_native, "lib", lambda: _NoLibrary())


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _mlp(T=16, h=32, f=64):
    return _bf(T, h), _bf(h, f), _bf(f), _bf(f, h)


@pytest.mark.parametrize("key,bad", [
    ("Y", lambda: _bf(16, 31)),                         # too small
    ("Y", lambda: _bf(32, 16).t()),                     # strided
    ("H", lambda: torch.zeros(16, 64)),                 # wrong dtype
    ("Z", lambda: _bf(15, 64)),
])
def test_mlp_fwd_rejects_bad_out(key, bad):
    x, a, b1, b = _mlp()
    with pytest.raises((ValueError, TypeError)):
        tps.mlp_shard_fwd(x, a, b1, b, tp_size=1, out={key: bad()})


def test_mlp_bwd_rejects_bad_out():
    x, a, _, b = _mlp()
    z, hh, dy = _bf(16, 64), _bf(16, 64), _bf(16, 32)
    with pytest.raises(ValueError):
        tps.mlp_shard_bwd(x, a, b, z, hh, dy, tp_size=1, out={"dA": torch.zeros(32, 63)})
    with pytest.raises(TypeError):
        tps.mlp_shard_bwd(x, a, b, z, hh, dy, tp_size=1, out={"dX": torch.zeros(16, 32)})   # fp32 dX for bf16


def test_workspace_must_be_contiguous_and_large_enough():
    x, a, _, b = _mlp()
    z, hh, dy = _bf(16, 64), _bf(16, 64), _bf(16, 32)
    with pytest.raises(ValueError):
        tps.mlp_shard_bwd(x, a, b, z, hh, dy, tp_size=1, workspace=torch.zeros(100, dtype=torch.uint8))
    strided = torch.zeros(4096, dtype=torch.uint8)[::2]
    with pytest.raises(ValueError):
        tps.mlp_shard_bwd(x, a, b, z, hh, dy, tp_size=1, workspace=strided)


def test_sp_edge_rejects_bad_out():
    x, g, dy = _bf(8, 32), _bf(32), _bf(8, 32)
    mean = rstd = torch.zeros(8)
    with pytest.raises(ValueError):
        tps.layernorm_bwd(x, g, mean, rstd, dy, out={"dX": _bf(8, 24)})
    with pytest.raises(ValueError):
        tps.bias_dropout_add_bwd(dy, p=0.1, seed=1, out=_bf(7, 32))
    with pytest.raises(TypeError):
        tps.bias_dropout_add_bwd(dy, p=0.1, seed=1, accumulate_into=_bf(32))     # bias grads are fp32
    with pytest.raises(ValueError):
        tps.bias_grad(dy, accumulate_into=torch.zeros(31))
