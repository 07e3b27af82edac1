"""CPU oracle (test infrastructure only): see minference_oracle."""
from .minference_oracle import *  # noqa: F401,F403
