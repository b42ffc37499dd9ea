"""float64 CPU oracle for fused RMSNorm + projection.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.
"""
from .flashnorm_oracle import *  # noqa: F401,F403
from .flashnorm_oracle import __all__  # noqa: F401
