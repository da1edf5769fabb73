"""fp64 CPU oracle for speculative-sampling verification (test infrastructure only)."""

from .specv_oracle import *  # noqa: F401,F403
from .specv_oracle import __all__  # noqa: F401
