"""Oracle package: plain float64 CPU reference of the Mixtral sparse MoE layer.

Test infrastructure only -- see ``oracle/moe_ref.py``.  The product path never
imports it.
"""
from .moe_ref import *  # noqa: F401,F403
