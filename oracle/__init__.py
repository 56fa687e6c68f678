"""fp64 CPU oracle of the FLASH layer forward (test infrastructure only; see flash_oracle)."""
from .flash_oracle import *  # noqa: F401,F403
from .flash_oracle import __all__  # noqa: F401
