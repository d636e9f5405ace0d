"""CPU float64 oracle (test infrastructure only; see ``duo_oracle``)."""
from .duo_oracle import *  # noqa: F401,F403
from . import duo_oracle  # noqa: F401
