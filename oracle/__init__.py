"""CPU oracle (test infrastructure only; never used by the product path)."""
from .qspec_oracle import *  # noqa: F401,F403
from .qspec_oracle import GROUP  # noqa: F401
