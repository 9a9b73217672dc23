"""CPU oracle of the MoE layer (test infrastructure only; see moe_oracle)."""
from . import moe_oracle  # noqa: F401
