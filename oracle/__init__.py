"""CPU oracle for the Hyena operator -- test infrastructure only (see hyena_oracle.py)."""
from .hyena_oracle import *  # noqa: F401,F403
