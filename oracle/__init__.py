"""CPU oracle (test infrastructure only; see twell_oracle.py's header)."""
from .twell_oracle import *  # noqa: F401,F403
