"""fp64 CPU oracle for exact attention (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library never does, and it shares no code with the
HIP path.  See ``oracle.attention`` for what is computed and where the source
pages state it, and ``oracle.brute`` for the decimal brute-force checks that
pin it.
"""
from .attention import *  # noqa: F401,F403
from . import attention, brute  # noqa: F401
