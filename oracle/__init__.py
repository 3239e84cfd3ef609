"""CPU oracle (test infrastructure only; see kq_oracle's header)."""
from .kq_oracle import *  # noqa: F401,F403
from .kq_oracle import __all__  # noqa: F401
