"""fp64 CPU oracle (test infrastructure only; see kvsel_oracle's docstring)."""
from .kvsel_oracle import *  # noqa: F401,F403
from .kvsel_oracle import __all__  # noqa: F401
