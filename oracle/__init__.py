"""fp64 CPU oracle of QUOKA's per-chunk hot path (test infrastructure only).

Only tests, the smoke check and the bench's CPU-baseline leg may use it; the
HIP library never imports or calls it.
"""
from .quoka import *  # noqa: F401,F403
from .quoka import __all__  # noqa: F401
