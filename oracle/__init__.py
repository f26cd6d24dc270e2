"""CPU oracle (test infrastructure only): see k2_oracle's header for what may import it."""
from .k2_oracle import *  # noqa: F401,F403
