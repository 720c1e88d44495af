"""fp64 CPU oracle for YaRN-RoPE blockwise attention.

TEST INFRASTRUCTURE: imported only by tests/, the smoke check and the
bench's CPU-baseline leg.  It shares no code with the HIP library, and the
library never imports it.
"""
from . import rope, attention  # noqa: F401
