"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This package only draws random numbers and stores them in the dtypes the
library consumes.  It holds none of the method's arithmetic (no scoring, no
selection, no attention).
"""
from .inputs import *  # noqa: F401,F403
