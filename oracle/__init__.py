"""fp64 CPU oracle for padded sigmoid attention (test infrastructure only)."""
from .sigattn_oracle import *  # noqa: F401,F403
