"""fp64 CPU oracle (test infrastructure only; see mk_oracle's header)."""
from .mk_oracle import *  # noqa: F401,F403
from .mk_oracle import __all__  # noqa: F401
