"""fp64 CPU oracle (test infrastructure only; see dsa_oracle's header)."""
from .dsa_oracle import *  # noqa: F401,F403
from .dsa_oracle import FORCE_DIAG, FORCE_SINK, RowSelection  # noqa: F401
