"""MI355X-native fused linear-recurrence scans for RL credit assignment.

The compute path is ``librlscan.so`` (hand-written HIP for gfx950, C ABI in
``include/rlscan.h``).  ``linear_recurrence_scan_amd.ops`` is a thin ctypes
binding with the same names; importing this package does not load the
library, so the seeded input generators in ``synth`` stay usable on machines
without a GPU.  Any op raises if the library or a GPU is missing: there is no
CPU fallback.
"""

__all__ = ["ops", "synth"]
