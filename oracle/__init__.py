"""CPU fp64 oracle (test infrastructure only; see cpa_oracle's header)."""
from . import cpa_oracle  # noqa: F401
