"""CPU oracle of the MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
anything from this package.  It shares no code with the GPU library.
"""
from . import moe  # noqa: F401
