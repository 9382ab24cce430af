"""MI355X (gfx950) compressed sparse attention (c4a / c128a DSA layer).

The compute path is the HIP library ``libdsa.so`` behind the C ABI in
``include/dsa.h``; ``sparse_long_context_c4a_amd._lib`` is its ctypes
binding and ``sparse_long_context_c4a_amd.layer`` marshals torch tensors
for a whole layer step.  ``configs`` holds the workload shapes and
``inputs`` the seeded synthetic input generator (CPU only).
"""

__all__ = ["configs", "inputs"]
