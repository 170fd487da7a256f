"""fp64 CPU oracle of the MSA routed-layer hot path (test infrastructure only)."""
from .msa_oracle import *  # noqa: F401,F403
