"""CPU oracle (test infrastructure only): see ``oracle.jssa_oracle``."""
from . import jssa_oracle  # noqa: F401
