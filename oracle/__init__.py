"""fp64 CPU oracle (test infrastructure only; see ``oracle.oracle``)."""
from .oracle import *  # noqa: F401,F403
from .oracle import __all__  # noqa: F401
