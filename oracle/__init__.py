"""Plain fp64 CPU oracle for the sink + rank-r decode state.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import or call anything here. The HIP library never routes
through it, and it shares no code with the HIP path.
"""
from .seed_oracle import *  # noqa: F401,F403
from .seed_oracle import __all__  # noqa: F401
