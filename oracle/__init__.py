"""CPU oracle (test infrastructure only; see sas_oracle's module docstring)."""
from . import sas_oracle  # noqa: F401
