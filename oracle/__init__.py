"""Float64 CPU oracle (test infrastructure only; see ``kvs_oracle``)."""
from . import kvs_oracle  # noqa: F401
