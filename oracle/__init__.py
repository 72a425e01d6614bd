"""CPU oracle for absorbed MLA (test infrastructure only; see mla_oracle.py)."""
from .mla_oracle import *  # noqa: F401,F403
