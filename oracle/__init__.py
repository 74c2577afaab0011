"""Plain fp64 CPU oracle for the double-binary-factorised product.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs
anything in this package; only the test-suite, the package's smoke check and
the benchmark's CPU-baseline leg do.  It shares no code with the HIP path.
"""
from .dbf_oracle import *  # noqa: F401,F403
from .dbf_oracle import __all__  # noqa: F401
