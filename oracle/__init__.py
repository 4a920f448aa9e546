"""CPU oracle for 64-token block-sparse attention (test infrastructure only; see vsa_oracle)."""
from .vsa_oracle import *  # noqa: F401,F403
from .vsa_oracle import BLOCK, LOG2E, ORDER_MIN_KV_BLOCKS  # noqa: F401
