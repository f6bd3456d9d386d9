"""CPU oracle (test infrastructure only; see area_oracle's header)."""
from .area_oracle import *  # noqa: F401,F403
