"""Float64 CPU oracle for FAVOR+ attention (test infrastructure only; the
product path never imports it)."""
from .favor_oracle import *  # noqa: F401,F403
from .favor_oracle import __all__ as _fa
from .projection import *  # noqa: F401,F403
from .projection import __all__ as _pa

__all__ = list(_fa) + list(_pa)
