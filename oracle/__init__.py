"""CPU oracle (test infrastructure only): see ``oracle.reference``."""
from .reference import *  # noqa: F401,F403
