"""fp64 CPU oracle (test infrastructure only; see psd_oracle)."""
from . import psd_oracle

__all__ = ["psd_oracle"]
