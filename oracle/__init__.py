"""fp64 CPU oracle for the BackLite hot path (test infrastructure only)."""
from . import backlite_oracle  # noqa: F401
