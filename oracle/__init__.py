"""CPU oracle of the MoE layer: test infrastructure only (see mok_oracle)."""
from .mok_oracle import *  # noqa: F401,F403
