"""CPU oracle for the MX hot path -- test infrastructure only (see mx_oracle)."""
from .mx_oracle import *  # noqa: F401,F403
from .mx_oracle import BLOCK, E2M1, E4M3  # noqa: F401
