"""CPU oracle (test infrastructure only; see vq_oracle's docstring)."""
from .vq_oracle import *  # noqa: F401,F403
from .vq_oracle import __all__  # noqa: F401
