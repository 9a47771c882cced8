"""CPU oracle (test infrastructure only): see oracle/moe_oracle.py."""
from .moe_oracle import *  # noqa: F401,F403
