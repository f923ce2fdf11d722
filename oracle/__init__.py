"""CPU oracle (test infrastructure only; see paro_oracle's header)."""
from .paro_oracle import *  # noqa: F401,F403
from .paro_oracle import GROUP, QMAX, SCALE_FLOOR  # noqa: F401
