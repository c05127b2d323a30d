"""CPU oracle of the intra-expert-sparse MoE layer (test infrastructure only;
see moe_oracle's header for who may use it)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import LayerResult, moe_layer  # noqa: F401
