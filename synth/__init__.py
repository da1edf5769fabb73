"""Seeded synthetic inputs shared by the HIP path's tests, the oracle and the benchmark."""

from .inputs import *  # noqa: F401,F403
from .inputs import __all__  # noqa: F401
