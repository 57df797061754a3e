"""CPU oracle for LCSA select + attend.  Test infrastructure only: the tests,
the smoke check and the bench's CPU-baseline leg use it; the library never
does."""
from .lcsa_oracle import *  # noqa: F401,F403
from .rope_oracle import *  # noqa: F401,F403
from .threshold_oracle import *  # noqa: F401,F403
