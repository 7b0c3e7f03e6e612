"""fp64 CPU oracle for the loss-scaling hook of the fp16 path.

TEST INFRASTRUCTURE ONLY. This module is imported by the test suite, by the
package smoke check and by the benchmark's CPU-baseline leg. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
it imports nothing from the product path.

Source: [TUT] "Megatron-LM：NVIDIA 的大规模并行训练方案", section "最佳实践与
调优建议" (mixed precision: train in fp16 or bf16) and "常见问题" (a loss that
turns NaN under fp16 is handled by dynamic loss scaling, or by switching to
bf16); [INTRO] "课程导入" 1.4.1 (fp32 master weights).  Dynamic loss scaling
multiplies the loss by S before the backward; the fp32 parameter gradients are
then multiplied by 1/S, and a step whose gradients hold an inf or NaN is
skipped (and S lowered).  The check-and-unscale of one gradient buffer is:
  g <- g * (1/S);  found <- found OR (any element of g is not finite).
"""
from __future__ import annotations

import numpy as np

__all__ = ["unscale_check_finite"]


def unscale_check_finite(grads, inv_scale: float):
    """Returns (grads * inv_scale in float64, whether any element is inf or NaN)."""
    g = np.asarray(grads, dtype=np.float64)
    return g * float(inv_scale), bool(not np.all(np.isfinite(g)))
