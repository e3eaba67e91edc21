"""CPU oracle for the MoE layer forward (test infrastructure; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
