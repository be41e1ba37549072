"""CPU oracle for the randomized Hadamard rotation + 4-bit quantisation path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It is a plain, slow, fp64 NumPy
restatement of the method's definition and shares no code, tables or
constants with the HIP library.
"""
from .rht_oracle import *  # noqa: F401,F403
from .rht_oracle import __all__  # noqa: F401
