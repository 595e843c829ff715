"""libs6: selective SSM scan (S6) for AMD MI355X.

The HIP library (libs6.so) is loaded on first use by the binding in
``selective_state_space_63_amd.s6``; ``synth`` holds the seeded workload
generator.
"""
from .s6 import S6Error, last_state, load_library, scan_fwd, state_update  # noqa: F401
