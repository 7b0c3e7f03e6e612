"""ctypes loader and prototypes for libtpshard.so (the C ABI in include/tpshard.h)."""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpshard.so")

TP_BF16, TP_FP32, TP_FP16 = 0, 1, 2
TP_ACT_NONE, TP_ACT_GELU = 0, 1
TP_OP_COLUMN_LINEAR_BWD, TP_OP_ROW_LINEAR_BWD, TP_OP_MLP_SHARD_BWD, TP_OP_BIAS_GRAD = 1, 2, 3, 4
TP_OP_ATTENTION_BWD, TP_OP_MLP_SHARD_BWD_RECOMPUTE, TP_OP_LAYERNORM_BWD, TP_OP_BIAS_DROPOUT_ADD_BWD = 5, 6, 7, 8
STATUS = {
    0: "TP_OK", -1: "TP_ERR_NULLPTR", -2: "TP_ERR_DIM", -3: "TP_ERR_TP_DIVISIBILITY",
    -4: "TP_ERR_ALIGNMENT", -5: "TP_ERR_DTYPE", -6: "TP_ERR_ALIAS", -7: "TP_ERR_WORKSPACE",
    -8: "TP_ERR_HIP", -9: "TP_ERR_ARG", -10: "TP_ERR_SCRATCH",
}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_fp = ctypes.c_void_p  # float* passed as an address

# name -> (restype, argtypes); mirrors include/tpshard.h
PROTOTYPES = {
    "tp_column_linear": (_i32, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "tp_row_linear": (_i32, [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _i32, _p]),
    "tp_mlp_shard_fwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i32, _p]),
    "tp_mlp_shard_bwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _fp, _fp, _fp, _fp, _p, _sz, _i32,
                                _i64, _i64, _i64, _i32, _i32, _p]),
    "tp_mlp_shard_bwd_recompute": (_i32, [_p, _p, _p, _p, _p, _p, _p, _fp, _fp, _fp, _fp, _p, _sz, _i32,
                                          _i64, _i64, _i64, _i32, _i32, _p]),
    "tp_mlp_shard_bwd_noalloc": (_i32, [_p, _p, _p, _p, _p, _p, _p, _fp, _fp, _fp, _fp, _i32,
                                        _i64, _i64, _i64, _i32, _i32, _p]),
    "tp_noalloc_scratch_bytes": (_sz, []),
    "tp_column_linear_bwd": (_i32, [_p, _p, _p, _p, _fp, _fp, _p, _sz, _i32, _i64, _i64, _i64, _i32, _i32, _p]),
    "tp_row_linear_bwd": (_i32, [_p, _p, _p, _p, _fp, _fp, _p, _sz, _i32, _i64, _i64, _i64, _i32, _i32, _p]),
    "tp_bias_grad": (_i32, [_p, _fp, _p, _sz, _i32, _i64, _i64, _i32, _p]),
    "tp_bias_gelu": (_i32, [_p, _p, _p, _i64, _i64, _i32, _p]),
    "tp_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i32, _i32]),
    "tp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tp_attention_fwd": (_i32, [_p, _p, _fp, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "tp_attention_bwd": (_i32, [_p, _p, _fp, _p, _p, _p, _sz, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "tp_layernorm_fwd": (_i32, [_p, _p, _p, _p, _fp, _fp, _i64, _i64, ctypes.c_float, _i32, _p]),
    "tp_layernorm_bwd": (_i32, [_p, _p, _fp, _fp, _p, _p, _fp, _fp, _p, _sz, _i32, _i64, _i64, _i32, _p]),
    "tp_bias_dropout_add_fwd": (_i32, [_p, _p, _p, _p, _i64, _i64, ctypes.c_double, ctypes.c_uint64,
                                       ctypes.c_uint64, _i32, _p]),
    "tp_bias_dropout_add_bwd": (_i32, [_p, _p, _fp, _p, _sz, _i32, _i64, _i64, ctypes.c_double, ctypes.c_uint64,
                                       ctypes.c_uint64, _i32, _p]),
    "tp_unscale_check_finite": (_i32, [_p, _i64, ctypes.c_float, _p, _p]),
    "tp_mfma_probe": (_i32, [_i32, _i32, _p, _p, _p]),
    "tp_wall_clock_rate_khz": (_i32, [ctypes.POINTER(_i32)]),
    "tp_trace_start": (_i32, [_i32]),
    "tp_trace_stop": (_i32, []),
    "tp_trace_num_kernels": (_i32, []),
    "tp_trace_kernel": (_i32, [_i32, ctypes.c_char_p, _sz, ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
}

_lib = None
_lock = threading.Lock()


class NativeLibraryMissing(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises NativeLibraryMissing when it is not built:
    there is no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise NativeLibraryMissing(
                    f"{LIB_PATH} is not built; run `python -m tensor_transformer_mlp_shard_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in PROTOTYPES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def check(status: int, what: str) -> None:
    if status != 0:
        text = lib().tp_status_string(status).decode()
        raise RuntimeError(f"{what}: {STATUS.get(status, status)} ({text})")
