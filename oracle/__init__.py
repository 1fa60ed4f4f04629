"""CPU oracle (test infrastructure only): see bifocal_oracle for what it computes and cites."""
from .bifocal_oracle import *  # noqa: F401,F403
from .bifocal_oracle import __all__  # noqa: F401
