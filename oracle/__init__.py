"""CPU oracle (test infrastructure only; never imported by the library path)."""
from .infini_oracle import *  # noqa: F401,F403
from .infini_oracle import EPS, backward, forward, forward_per_token, segment_unit, state_sweep  # noqa: F401
