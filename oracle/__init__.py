"""fp64 CPU oracle of the flow-matching Euler denoise loop.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import anything under this directory; the GPU library
never calls, links or loads it, and it shares no code with the library.
"""
from .fm_oracle import *  # noqa: F401,F403
from .fm_oracle import __all__  # noqa: F401
