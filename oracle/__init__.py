"""fp64 CPU oracle (test infrastructure only; never used by the product path).

See oracle/tp_shard.py (linear shards, MLP) and oracle/attention.py (core
attention on the local heads) for the definitions and their sources.
"""
from .tp_shard import *  # noqa: F401,F403
from .tp_shard import __all__ as _tp_all
from .attention import *  # noqa: F401,F403
from .attention import __all__ as _attn_all

__all__ = list(_tp_all) + list(_attn_all)
