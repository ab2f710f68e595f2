"""fp64 CPU oracle of the MLA forward (test infrastructure).

Only tests/, smoke() in __graft_entry__.py and bench.py's cpu_baseline leg may
import this package. It shares no code with the HIP library and never imports it.
"""
from . import fp8, mask, mla  # noqa: F401
