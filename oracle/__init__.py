"""CPU oracle (test infrastructure only; see cfm_oracle)."""
from .cfm_oracle import *  # noqa: F401,F403
