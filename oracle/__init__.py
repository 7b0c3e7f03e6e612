"""fp64 CPU oracle (test infrastructure only; never used by the product path).

See oracle/tp_shard.py (linear shards, MLP), oracle/attention.py (core
attention on the local heads) and oracle/sp_edge.py (LayerNorm, bias + dropout
+ residual, Philox4x32-10) and oracle/loss_scale.py (loss-scaling check) for
the definitions and their sources.
"""
from .tp_shard import *  # noqa: F401,F403
from .tp_shard import __all__ as _tp_all
from .attention import *  # noqa: F401,F403
from .attention import __all__ as _attn_all

from .sp_edge import *  # noqa: F401,F403
from .sp_edge import __all__ as _sp_all

from .loss_scale import *  # noqa: F401,F403
from .loss_scale import __all__ as _ls_all

__all__ = list(_tp_all) + list(_attn_all) + list(_sp_all) + list(_ls_all)
