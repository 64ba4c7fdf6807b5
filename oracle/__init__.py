"""CPU oracle of the sparse-MoE layer forward (test infrastructure; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
