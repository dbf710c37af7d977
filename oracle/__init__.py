"""fp64 CPU oracle (test infrastructure; see tp_oracle's header)."""
from .tp_oracle import *  # noqa: F401,F403
from .tp_oracle import __all__  # noqa: F401
