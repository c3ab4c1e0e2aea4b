"""CPU oracle (test infrastructure only; see ``sa_oracle``)."""
from .sa_oracle import *  # noqa: F401,F403
from .sa_oracle import DENSE, REUSE, SPARSE  # noqa: F401
