"""CPU oracle for CA-SGD (test infrastructure only; see casgd_oracle)."""
from .casgd_oracle import *  # noqa: F401,F403
from . import casgd_oracle  # noqa: F401
