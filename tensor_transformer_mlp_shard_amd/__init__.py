"""MI355X-native tensor-parallel Transformer shard: Python binding of libtpshard.so.

Each function marshals torch CUDA tensors (device memory and the current HIP
stream) into one call of the C ABI declared in include/tpshard.h; every step of
the computation runs in the library's HIP kernels.  Outputs are allocated with
``torch.empty`` on the inputs' device.  There is no fallback: without the built
library every call raises.

Shapes (rank i of a TP group of size p; weights are [in x out]):
  column_linear   X[T x K], W_i[K x N/p]           -> Y_i[T x N/p]
  row_linear      X_i[T x K/p], W_i[K/p x N]       -> Y_i[T x N] (partial)
  mlp_shard_fwd   X[T x h], A_i[h x f], B_i[f x h] -> Z_i, H_i [T x f], Y_i[T x h]
  *_bwd           the matching gradients; parameter gradients are fp32.
"""
from __future__ import annotations

import ctypes

import torch

from . import _native
from ._native import NativeLibraryMissing  # noqa: F401

__all__ = [
    "column_linear", "row_linear", "mlp_shard_fwd", "mlp_shard_bwd", "column_linear_bwd",
    "row_linear_bwd", "bias_grad", "bias_gelu", "workspace_size", "trace_start", "trace_stop",
    "attention_fwd", "attention_bwd", "layernorm_fwd", "layernorm_bwd", "bias_dropout_add_fwd",
    "bias_dropout_add_bwd", "unscale_check_finite", "mfma_probe", "library_path", "NativeLibraryMissing",
    "mlp_shard_bwd_noalloc", "noalloc_scratch_bytes",
]

_DT = {torch.bfloat16: _native.TP_BF16, torch.float32: _native.TP_FP32, torch.float16: _native.TP_FP16}


def library_path() -> str:
    _native.lib()
    return _native.LIB_PATH


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16, float16 or float32")
    return _DT[t.dtype]


def _require_gpu(name, t):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")


def _check(name, t, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    _require_gpu(name, t)
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(out, key, shape, dtype, device):
    """out[key] checked like an input (shape, dtype, device, contiguity), or a
    new tensor when the caller gave none."""
    t = out.get(key)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _check(f"out[{key}]", t, shape, dtype, device)
    return t


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_size(op: int, T: int, d_in: int, d_out: int, tp_size: int, dtype: torch.dtype) -> int:
    return int(_native.lib().tp_workspace_size(op, T, d_in, d_out, tp_size, _DT[dtype]))


def _workspace(op, T, d_in, d_out, tp_size, dtype, device, given):
    need = workspace_size(op, T, d_in, d_out, tp_size, dtype)
    if given is not None:
        if (given.device != device or not given.is_contiguous()
                or given.numel() * given.element_size() < need):
            raise ValueError(f"workspace needs {need} contiguous bytes on {device}")
        return given
    return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


def column_linear(x, w_i, b_i=None, *, tp_size: int, act: str = "none", save_z: bool = False):
    """Column-parallel linear (rank's shard).  Returns Y_i, or (Y_i, Z_i) when
    act == "gelu" and save_z."""
    T, K = x.shape
    n = w_i.shape[1]
    dt = x.dtype
    _check("x", x, (T, K), dt, x.device)
    _check("w_i", w_i, (K, n), dt, x.device)
    if b_i is not None:
        _check("b_i", b_i, (n,), dt, x.device)
    if act not in ("none", "gelu"):
        raise ValueError("act must be 'none' or 'gelu'")
    if save_z and act != "gelu":
        raise ValueError("save_z needs act='gelu'")
    y = torch.empty((T, n), dtype=dt, device=x.device)
    z = torch.empty((T, n), dtype=dt, device=x.device) if save_z else None
    st = _native.lib().tp_column_linear(
        _ptr(x), _ptr(w_i), _ptr(b_i), _ptr(y), _ptr(z), T, K, n * tp_size, tp_size,
        _native.TP_ACT_GELU if act == "gelu" else _native.TP_ACT_NONE, _dtype_code(x), _stream(x.device))
    _native.check(st, "tp_column_linear")
    return (y, z) if save_z else y


def row_linear(x_i, w_i, b=None, *, tp_size: int):
    """Row-parallel linear: the rank's partial X_i W_i (+ b)."""
    T, k = x_i.shape
    N = w_i.shape[1]
    dt = x_i.dtype
    _check("x_i", x_i, (T, k), dt, x_i.device)
    _check("w_i", w_i, (k, N), dt, x_i.device)
    if b is not None:
        _check("b", b, (N,), dt, x_i.device)
    y = torch.empty((T, N), dtype=dt, device=x_i.device)
    st = _native.lib().tp_row_linear(_ptr(x_i), _ptr(w_i), _ptr(b), _ptr(y), T, k * tp_size, N, tp_size,
                                     _dtype_code(x_i), _stream(x_i.device))
    _native.check(st, "tp_row_linear")
    return y


def mlp_shard_fwd(x, a_i, b1_i, b_i, *, tp_size: int, save_z: bool = True, out=None):
    """MLP shard forward.  Returns (Z_i or None, H_i, Y_i).  ``out`` may hold
    preallocated "Z", "H", "Y" tensors."""
    T, h = x.shape
    f = a_i.shape[1]
    dt = x.dtype
    dev = x.device
    _check("x", x, (T, h), dt, dev)
    _check("a_i", a_i, (h, f), dt, dev)
    _check("b_i", b_i, (f, h), dt, dev)
    if b1_i is not None:
        _check("b1_i", b1_i, (f,), dt, dev)
    out = out or {}
    z = _out(out, "Z", (T, f), dt, dev) if save_z else None
    hh = _out(out, "H", (T, f), dt, dev)
    y = _out(out, "Y", (T, h), dt, dev)
    st = _native.lib().tp_mlp_shard_fwd(_ptr(x), _ptr(a_i), _ptr(b1_i), _ptr(b_i), _ptr(z), _ptr(hh), _ptr(y),
                                        T, h, f * tp_size, tp_size, _dtype_code(x), _stream(dev))
    _native.check(st, "tp_mlp_shard_fwd")
    return z, hh, y


def mlp_shard_bwd(x, a_i, b_i, z_i, h_i, dy, *, tp_size: int, want_db1: bool = True, want_db2: bool = False,
                  accumulate: bool = False, out=None, workspace=None, recompute: bool = False, b1_i=None):
    """MLP shard backward.  Returns dict(dX, dA, db1, dB, db2) (db1 / db2 None
    unless wanted).  With ``accumulate`` the fp32 parameter gradients in ``out``
    ("dA", "dB", "db1", "db2") are added to instead of overwritten.

    ``recompute=True`` selects the selective-recompute form
    (tp_mlp_shard_bwd_recompute): ``h_i`` must be None; with ``z_i`` given, H is
    recomputed from it; with ``z_i`` None too, Z and H are recomputed from
    ``x`` by the fc1 GEMM with bias ``b1_i``."""
    T, h = x.shape
    f = a_i.shape[1]
    dt = x.dtype
    dev = x.device
    checks = [("x", x, (T, h)), ("a_i", a_i, (h, f)), ("b_i", b_i, (f, h)), ("dy", dy, (T, h))]
    if recompute:
        if h_i is not None:
            raise ValueError("recompute=True takes no saved h_i")
        if z_i is not None:
            checks.append(("z_i", z_i, (T, f)))
        if b1_i is not None:
            checks.append(("b1_i", b1_i, (f,)))
    else:
        checks += [("z_i", z_i, (T, f)), ("h_i", h_i, (T, f))]
    for name, t, shp in checks:
        _check(name, t, shp, dt, dev)
    out = dict(out or {})
    if accumulate:
        for k in ("dA", "dB") + (("db1",) if want_db1 else ()) + (("db2",) if want_db2 else ()):
            if out.get(k) is None:
                raise ValueError(f"accumulate needs out[{k!r}]")

    def get(k, shape, dtype):
        t = out.get(k)
        if t is None:
            return torch.empty(shape, dtype=dtype, device=dev)
        _check(f"out[{k}]", t, shape, dtype, dev)
        return t

    dX = get("dX", (T, h), dt)
    dA = get("dA", (h, f), torch.float32)
    dB = get("dB", (f, h), torch.float32)
    db1 = get("db1", (f,), torch.float32) if want_db1 else None
    db2 = get("db2", (h,), torch.float32) if want_db2 else None
    if recompute:
        ws = _workspace(_native.TP_OP_MLP_SHARD_BWD_RECOMPUTE, T, h, f * tp_size, tp_size, dt, dev, workspace)
        st = _native.lib().tp_mlp_shard_bwd_recompute(
            _ptr(x), _ptr(a_i), _ptr(b1_i), _ptr(b_i), _ptr(z_i), _ptr(dy), _ptr(dX), _ptr(dA), _ptr(db1),
            _ptr(dB), _ptr(db2), _ptr(ws), _nbytes(ws), int(accumulate), T, h, f * tp_size, tp_size,
            _dtype_code(x), _stream(dev))
        _native.check(st, "tp_mlp_shard_bwd_recompute")
    else:
        ws = _workspace(_native.TP_OP_MLP_SHARD_BWD, T, h, f * tp_size, tp_size, dt, dev, workspace)
        st = _native.lib().tp_mlp_shard_bwd(
            _ptr(x), _ptr(a_i), _ptr(b_i), _ptr(z_i), _ptr(h_i), _ptr(dy), _ptr(dX), _ptr(dA), _ptr(db1),
            _ptr(dB), _ptr(db2), _ptr(ws), _nbytes(ws), int(accumulate), T, h, f * tp_size, tp_size,
            _dtype_code(x), _stream(dev))
        _native.check(st, "tp_mlp_shard_bwd")
    return {"dX": dX, "dA": dA, "db1": db1, "dB": dB, "db2": db2}


def noalloc_scratch_bytes() -> int:
    """Bytes of the static device scratch of mlp_shard_bwd_noalloc."""
    return int(_native.lib().tp_noalloc_scratch_bytes())


def mlp_shard_bwd_noalloc(x, a_i, b_i, z_i, h_i, dy, *, tp_size: int, out, want_db1: bool = True,
                          want_db2: bool = False, accumulate: bool = False):
    """MLP shard backward through tp_mlp_shard_bwd_noalloc: the same results as
    mlp_shard_bwd with its scratch in the library's static device array, for
    callers that cannot allocate.  Nothing is allocated here either: ``out``
    must hold "dX", "dA", "dB" (and "db1" / "db2" when wanted).  Calls that
    overlap on one GPU race on that array."""
    T, h = x.shape
    f = a_i.shape[1]
    dt = x.dtype
    dev = x.device
    for name, t, shp in (("x", x, (T, h)), ("a_i", a_i, (h, f)), ("b_i", b_i, (f, h)), ("z_i", z_i, (T, f)),
                         ("h_i", h_i, (T, f)), ("dy", dy, (T, h))):
        _check(name, t, shp, dt, dev)
    need = [("dX", (T, h), dt), ("dA", (h, f), torch.float32), ("dB", (f, h), torch.float32)]
    need += [("db1", (f,), torch.float32)] if want_db1 else []
    need += [("db2", (h,), torch.float32)] if want_db2 else []
    for k, shp, tdt in need:
        if out.get(k) is None:
            raise ValueError(f"mlp_shard_bwd_noalloc allocates nothing: out[{k!r}] is required")
        _check(f"out[{k}]", out[k], shp, tdt, dev)
    db1 = out["db1"] if want_db1 else None
    db2 = out["db2"] if want_db2 else None
    st = _native.lib().tp_mlp_shard_bwd_noalloc(
        _ptr(x), _ptr(a_i), _ptr(b_i), _ptr(z_i), _ptr(h_i), _ptr(dy), _ptr(out["dX"]), _ptr(out["dA"]), _ptr(db1),
        _ptr(out["dB"]), _ptr(db2), int(accumulate), T, h, f * tp_size, tp_size, _dtype_code(x), _stream(dev))
    _native.check(st, "tp_mlp_shard_bwd_noalloc")
    return out


def _linear_bwd(fn_name, op, x, w, dy, T, K, N, tp_size, dx_shape, want_db, accumulate, out, workspace):
    dev = x.device
    dt = x.dtype
    out = dict(out or {})
    if accumulate:
        for k in ("dW",) + (("db",) if want_db else ()):
            if out.get(k) is None:
                raise ValueError(f"accumulate needs out[{k!r}]")

    def get(k, shape, dtype):
        t = out.get(k)
        if t is None:
            return torch.empty(shape, dtype=dtype, device=dev)
        _check(f"out[{k}]", t, shape, dtype, dev)
        return t

    dX = get("dX", dx_shape, dt)
    dW = get("dW", tuple(w.shape), torch.float32)
    db = get("db", (dy.shape[1],), torch.float32) if want_db else None
    ws = _workspace(op, T, K, N, tp_size, dt, dev, workspace) if want_db else None
    fn = getattr(_native.lib(), fn_name)
    st = fn(_ptr(x), _ptr(w), _ptr(dy), _ptr(dX), _ptr(dW), _ptr(db), _ptr(ws), 0 if ws is None else _nbytes(ws),
            int(accumulate), T, K, N, tp_size, _dtype_code(x), _stream(dev))
    _native.check(st, fn_name)
    return {"dX": dX, "dW": dW, "db": db}


def column_linear_bwd(x, w_i, dy_i, *, tp_size: int, want_db: bool = True, accumulate: bool = False, out=None,
                      workspace=None):
    """Column-parallel linear backward: dict(dX (partial), dW, db)."""
    T, K = x.shape
    n = w_i.shape[1]
    dt = x.dtype
    _check("x", x, (T, K), dt, x.device)
    _check("w_i", w_i, (K, n), dt, x.device)
    _check("dy_i", dy_i, (T, n), dt, x.device)
    return _linear_bwd("tp_column_linear_bwd", _native.TP_OP_COLUMN_LINEAR_BWD, x, w_i, dy_i, T, K, n * tp_size,
                       tp_size, (T, K), want_db, accumulate, out, workspace)


def row_linear_bwd(x_i, w_i, dy, *, tp_size: int, want_db: bool = True, accumulate: bool = False, out=None,
                   workspace=None):
    """Row-parallel linear backward: dict(dX (this rank's input block), dW, db)."""
    T, k = x_i.shape
    N = w_i.shape[1]
    dt = x_i.dtype
    _check("x_i", x_i, (T, k), dt, x_i.device)
    _check("w_i", w_i, (k, N), dt, x_i.device)
    _check("dy", dy, (T, N), dt, x_i.device)
    return _linear_bwd("tp_row_linear_bwd", _native.TP_OP_ROW_LINEAR_BWD, x_i, w_i, dy, T, k * tp_size, N,
                       tp_size, (T, k), want_db, accumulate, out, workspace)


def bias_grad(dy, *, accumulate_into=None, workspace=None):
    """Sum over tokens of dy [T x N] -> fp32 [N]."""
    T, N = dy.shape
    dev = dy.device
    _check("dy", dy, (T, N), dy.dtype, dev)
    if accumulate_into is not None:
        _check("accumulate_into", accumulate_into, (N,), torch.float32, dev)
    db = accumulate_into if accumulate_into is not None else torch.empty((N,), dtype=torch.float32, device=dev)
    ws = _workspace(_native.TP_OP_BIAS_GRAD, T, N, 0, 1, dy.dtype, dev, workspace)
    st = _native.lib().tp_bias_grad(_ptr(dy), _ptr(db), _ptr(ws), _nbytes(ws), int(accumulate_into is not None),
                                    T, N, _dtype_code(dy), _stream(dev))
    _native.check(st, "tp_bias_grad")
    return db


def bias_gelu(z, b=None):
    """Unfused H = GeLU(Z + b)."""
    T, N = z.shape
    _check("z", z, (T, N), z.dtype, z.device)
    if b is not None:
        _check("b", b, (N,), z.dtype, z.device)
    hh = torch.empty_like(z)
    st = _native.lib().tp_bias_gelu(_ptr(z), _ptr(b), _ptr(hh), T, N, _dtype_code(z), _stream(z.device))
    _native.check(st, "tp_bias_gelu")
    return hh


def attention_fwd(qkv, *, seq: int, heads: int, head_dim: int, tp_size: int, causal: bool = True,
                  save_lse: bool = True, out=None):
    """Core attention on the rank's heads: qkv [T x 3*Hl*d] -> (O [T x Hl*d], lse [Hl x T] or None)."""
    T, W = qkv.shape
    hl = heads // tp_size if tp_size > 0 else 0
    dev = qkv.device
    _check("qkv", qkv, (T, 3 * hl * head_dim), torch.bfloat16, dev)
    o = out if out is not None else torch.empty((T, hl * head_dim), dtype=torch.bfloat16, device=dev)
    _check("out", o, (T, hl * head_dim), torch.bfloat16, dev)
    lse = torch.empty((hl, T), dtype=torch.float32, device=dev) if save_lse else None
    st = _native.lib().tp_attention_fwd(_ptr(qkv), _ptr(o), _ptr(lse), T, seq, heads, head_dim, tp_size,
                                        int(causal), _native.TP_BF16, _stream(dev))
    _native.check(st, "tp_attention_fwd")
    return o, lse


def attention_bwd(qkv, o, lse, dout, *, seq: int, heads: int, head_dim: int, tp_size: int, causal: bool = True,
                  out=None, workspace=None):
    """Backward of attention_fwd: -> dQKV [T x 3*Hl*d] (same [Q | K | V] layout as qkv)."""
    T = qkv.shape[0]
    hl = heads // tp_size if tp_size > 0 else 0
    dev = qkv.device
    w = hl * head_dim
    _check("qkv", qkv, (T, 3 * w), torch.bfloat16, dev)
    _check("o", o, (T, w), torch.bfloat16, dev)
    _check("lse", lse, (hl, T), torch.float32, dev)
    _check("dout", dout, (T, w), torch.bfloat16, dev)
    dq = out if out is not None else torch.empty((T, 3 * w), dtype=torch.bfloat16, device=dev)
    _check("out", dq, (T, 3 * w), torch.bfloat16, dev)
    ws = _workspace(_native.TP_OP_ATTENTION_BWD, T, heads, head_dim, tp_size, torch.bfloat16, dev, workspace)
    st = _native.lib().tp_attention_bwd(_ptr(qkv), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(ws),
                                        _nbytes(ws), T, seq, heads, head_dim, tp_size,
                                        int(causal), _native.TP_BF16, _stream(dev))
    _native.check(st, "tp_attention_bwd")
    return dq


def layernorm_fwd(x, gamma, beta=None, *, eps: float = 1e-5, save_stats: bool = True, out=None):
    """LayerNorm over the last dimension of x [rows x h] -> (y, mean or None, rstd or None)."""
    rows, h = x.shape
    dev, dt = x.device, x.dtype
    _check("x", x, (rows, h), dt, dev)
    _check("gamma", gamma, (h,), dt, dev)
    if beta is not None:
        _check("beta", beta, (h,), dt, dev)
    y = out if out is not None else torch.empty_like(x)
    _check("out", y, (rows, h), dt, dev)
    mean = torch.empty((rows,), dtype=torch.float32, device=dev) if save_stats else None
    rstd = torch.empty((rows,), dtype=torch.float32, device=dev) if save_stats else None
    st = _native.lib().tp_layernorm_fwd(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), rows, h,
                                        float(eps), _dtype_code(x), _stream(dev))
    _native.check(st, "tp_layernorm_fwd")
    return y, mean, rstd


def layernorm_bwd(x, gamma, mean, rstd, dy, *, want_dbeta: bool = True, accumulate: bool = False, out=None,
                  workspace=None):
    """LayerNorm backward -> dict(dX, dgamma, dbeta)."""
    rows, h = x.shape
    dev, dt = x.device, x.dtype
    for name, t, shp, tdt in (("x", x, (rows, h), dt), ("gamma", gamma, (h,), dt), ("dy", dy, (rows, h), dt),
                              ("mean", mean, (rows,), torch.float32), ("rstd", rstd, (rows,), torch.float32)):
        _check(name, t, shp, tdt, dev)
    out = dict(out or {})

    def get(k, shape, dtype):
        t = out.get(k)
        if t is None:
            if accumulate:
                raise ValueError(f"accumulate needs out[{k!r}]")
            return torch.empty(shape, dtype=dtype, device=dev)
        _check(f"out[{k}]", t, shape, dtype, dev)
        return t

    dX = _out(out, "dX", (rows, h), dt, dev)
    dg = get("dgamma", (h,), torch.float32)
    db = get("dbeta", (h,), torch.float32) if want_dbeta else None
    ws = _workspace(_native.TP_OP_LAYERNORM_BWD, rows, h, 0, 1, dt, dev, workspace)
    st = _native.lib().tp_layernorm_bwd(_ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dy), _ptr(dX), _ptr(dg),
                                        _ptr(db), _ptr(ws), _nbytes(ws), int(accumulate), rows, h, _dtype_code(x),
                                        _stream(dev))
    _native.check(st, "tp_layernorm_bwd")
    return {"dX": dX, "dgamma": dg, "dbeta": db}


def bias_dropout_add_fwd(y, b, residual, *, p: float, seed: int, offset: int = 0, out=None):
    """residual + dropout(y + b) with the Philox4x32-10 keep rule -> out."""
    rows, h = y.shape
    dev, dt = y.device, y.dtype
    _check("y", y, (rows, h), dt, dev)
    _check("residual", residual, (rows, h), dt, dev)
    if b is not None:
        _check("b", b, (h,), dt, dev)
    o = out if out is not None else torch.empty_like(y)
    _check("out", o, (rows, h), dt, dev)
    st = _native.lib().tp_bias_dropout_add_fwd(_ptr(y), _ptr(b), _ptr(residual), _ptr(o), rows, h, float(p),
                                               int(seed), int(offset), _dtype_code(y), _stream(dev))
    _native.check(st, "tp_bias_dropout_add_fwd")
    return o


def bias_dropout_add_bwd(dout, *, p: float, seed: int, offset: int = 0, want_db: bool = True, accumulate_into=None,
                         out=None, workspace=None):
    """Backward of bias_dropout_add_fwd -> (dY, db or None); the residual's gradient is dout."""
    rows, h = dout.shape
    dev, dt = dout.device, dout.dtype
    _check("dout", dout, (rows, h), dt, dev)
    dY = out if out is not None else torch.empty_like(dout)
    _check("out", dY, (rows, h), dt, dev)
    if accumulate_into is not None:
        _check("accumulate_into", accumulate_into, (h,), torch.float32, dev)
    db = accumulate_into if accumulate_into is not None else (
        torch.empty((h,), dtype=torch.float32, device=dev) if want_db else None)
    ws = _workspace(_native.TP_OP_BIAS_DROPOUT_ADD_BWD, rows, h, 0, 1, dt, dev, workspace) if db is not None else None
    st = _native.lib().tp_bias_dropout_add_bwd(_ptr(dout), _ptr(dY), _ptr(db), _ptr(ws),
                                               _nbytes(ws) if ws is not None else 0, int(accumulate_into is not None),
                                               rows, h, float(p), int(seed), int(offset), _dtype_code(dout),
                                               _stream(dev))
    _native.check(st, "tp_bias_dropout_add_bwd")
    return dY, db


def unscale_check_finite(grads, inv_scale: float, found):
    """grads (fp32, contiguous) *= inv_scale in place; sets found (int32 [1] on the
    device) to 1 if any element is inf or NaN.  found is never cleared here."""
    _check("grads", grads, tuple(grads.shape), torch.float32, grads.device)
    _check("found", found, (1,), torch.int32, grads.device)
    st = _native.lib().tp_unscale_check_finite(_ptr(grads), grads.numel(), float(inv_scale), _ptr(found),
                                               _stream(grads.device))
    _native.check(st, "tp_unscale_check_finite")


def trace_start(max_launches: int = 4096) -> None:
    _native.check(_native.lib().tp_trace_start(max_launches), "tp_trace_start")


def trace_stop():
    """Stop the trace; returns a list of dicts(name, launches, total_ms, flops, bytes)."""
    L = _native.lib()
    _native.check(L.tp_trace_stop(), "tp_trace_stop")
    out = []
    buf = ctypes.create_string_buffer(256)
    for i in range(L.tp_trace_num_kernels()):
        n = ctypes.c_int64()
        ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        _native.check(L.tp_trace_kernel(i, buf, 256, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl),
                                        ctypes.byref(by)), "tp_trace_kernel")
        out.append({"name": buf.value.decode(), "launches": n.value, "total_ms": ms.value, "flops": fl.value,
                    "bytes": by.value})
    return out


MFMA_FLOP = 2 * 32 * 32 * 16   # one bf16 32x32x16 MFMA
FLOP_PER_CU_CLK = 4096         # dense bf16 matrix-core rate of one compute unit


def mfma_probe(iters: int = 100000, blocks: int | None = None, device=None) -> dict:
    """Run the register-only MFMA probe once and return what it sustained:
    TFLOP/s over the kernel's event time, the mean and minimum shader clock
    (GHz) over the workgroups, and the matrix-pipe busy fraction implied by
    the cycle counts (1.0 when every SIMD issues one MFMA per 32 cycles).
    ``blocks`` defaults to two 4-wave workgroups per compute unit."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus if blocks is None else blocks
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    ticks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    L = _native.lib()
    khz = ctypes.c_int32()
    with torch.cuda.device(dev):
        _native.check(L.tp_wall_clock_rate_khz(ctypes.byref(khz)), "tp_wall_clock_rate_khz")
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        _native.check(L.tp_mfma_probe(blocks, iters, _ptr(sink), _ptr(ticks), _stream(dev)), "tp_mfma_probe")
        stop.record()
        stop.synchronize()
    ms = start.elapsed_time(stop)
    t = ticks.view(blocks, 2).cpu().double()
    cycles, wall_s = t[:, 0], t[:, 1] / (khz.value * 1e3)
    ghz = cycles / wall_s / 1e9
    flops = float(blocks) * 4 * 16 * iters * MFMA_FLOP
    # MFMAs each SIMD issued, over the cycles the slowest workgroup took
    waves_per_simd = blocks * 4 / (4 * cus)
    busy = waves_per_simd * 16 * iters * 32 / float(cycles.max())
    return {"tflops": flops / (ms * 1e-3) / 1e12, "ms": ms, "clock_ghz_mean": float(ghz.mean()),
            "clock_ghz_min": float(ghz.min()), "mfma_busy": busy, "blocks": blocks, "iters": iters,
            "compute_units": cus, "finite": bool(torch.isfinite(sink).all().item())}
