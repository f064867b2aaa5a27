"""Oracle package — test infrastructure only (see dg_oracle's header)."""
from . import dg_oracle  # noqa: F401
