"""fp64 CPU oracle (test infrastructure only; never used by the product path).

See oracle/tp_shard.py for the definitions and their sources.
"""
from .tp_shard import *  # noqa: F401,F403
from .tp_shard import __all__  # noqa: F401
