"""CPU oracle (test infrastructure only): see tis_oracle."""
from .tis_oracle import widen, tree_build, tree_route, tree_attend, decode  # noqa: F401
