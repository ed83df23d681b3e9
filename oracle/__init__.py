"""CPU oracle (test infrastructure only; see sk_oracle's module docstring)."""
from .sk_oracle import *  # noqa: F401,F403
from . import sk_oracle  # noqa: F401
