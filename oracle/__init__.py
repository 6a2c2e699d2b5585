"""CPU oracle (test infrastructure only; see sfi_oracle's header)."""
from . import sfi_oracle  # noqa: F401
