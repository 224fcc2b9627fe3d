"""fp64 CPU oracle for the MoBA prefill forward (test infrastructure only)."""
from .moba_oracle import *  # noqa: F401,F403
