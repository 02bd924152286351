"""CPU oracle of the MoE expert layer (test infrastructure only; see moe_oracle's header)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
