"""fp64 CPU oracle (test infrastructure only; never used by the product path).

See oracle/tp_shard.py (linear shards, MLP), oracle/attention.py (core
attention on the local heads) and oracle/sp_edge.py (LayerNorm, bias + dropout
+ residual, Philox4x32-10) for the definitions and their sources.
"""
from .tp_shard import *  # noqa: F401,F403
from .tp_shard import __all__ as _tp_all
from .attention import *  # noqa: F401,F403
from .attention import __all__ as _attn_all

from .sp_edge import *  # noqa: F401,F403
from .sp_edge import __all__ as _sp_all

__all__ = list(_tp_all) + list(_attn_all) + list(_sp_all)
