"""CPU oracle (test infrastructure only): see rtp_oracle.py."""
from .rtp_oracle import *  # noqa: F401,F403
