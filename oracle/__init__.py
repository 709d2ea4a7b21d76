"""CPU oracle (test infrastructure only; see ``sva_oracle``)."""
from .sva_oracle import *  # noqa: F401,F403
from .sva_oracle import Geometry, SVA_DENSE, SVA_KEEP_SAME_FRAME  # noqa: F401
