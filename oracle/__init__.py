"""CPU oracle (test infrastructure only; see dg_oracle's module docstring)."""
from .dg_oracle import *  # noqa: F401,F403
