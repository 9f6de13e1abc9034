"""CPU oracle package (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. It is a plain float64 implementation of the fused NVFP4 W4A4
operator written from the definition; it shares no code with the HIP path.
"""
from .w4a4_ref import *  # noqa: F401,F403
from .w4a4_ref import __all__  # noqa: F401
