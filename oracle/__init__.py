"""CPU oracle (test infrastructure only; never imported by the library)."""
from .reference import *  # noqa: F401,F403
