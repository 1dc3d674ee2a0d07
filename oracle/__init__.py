"""fp64 CPU oracle of the BRA forward pass (test infrastructure only; see
bra_oracle's header)."""
from .bra_oracle import *  # noqa: F401,F403
from .bra_oracle import __all__  # noqa: F401
