"""fp64 CPU oracle for MLA decode: test infrastructure only (see mla_oracle's header)."""
from .mla_oracle import *  # noqa: F401,F403
