"""Float64 CPU oracle (test infrastructure only; see egs_oracle.py)."""
from .egs_oracle import *  # noqa: F401,F403
