"""CPU oracle (test infrastructure only; see dyadic24.py's header)."""
from . import dyadic24  # noqa: F401
