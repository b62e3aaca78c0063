"""CPU oracle (test infrastructure only; see kvq_oracle.py's header)."""
from . import kvq_oracle  # noqa: F401
