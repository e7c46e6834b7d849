"""CPU float64 oracle (test infrastructure only; never imported by the product path)."""
from . import bd_oracle  # noqa: F401
