"""CPU oracle (test infrastructure only; see gtq_oracle's header)."""
from .gtq_oracle import *  # noqa: F401,F403
from . import gtq_oracle  # noqa: F401
