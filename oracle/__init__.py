"""fp64 CPU oracle (test infrastructure only; never used by the GPU library)."""
from .moe_oracle import *  # noqa: F401,F403
