"""CPU oracle of the MoE layer (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import NEAR_TIE  # noqa: F401
