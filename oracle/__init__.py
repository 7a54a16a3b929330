"""CPU oracle of the KVarN hot path (test infrastructure only)."""
from .kvarn_oracle import *  # noqa: F401,F403
from .kvarn_oracle import GROUP, SINK, TAIL_CAP, SINKHORN_ITERS  # noqa: F401
