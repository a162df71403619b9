"""CPU oracle (test infrastructure only; see bitlinear_oracle)."""
from .bitlinear_oracle import *  # noqa: F401,F403
