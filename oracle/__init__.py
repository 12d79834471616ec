"""CPU oracle of the routed-MoE layer (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
