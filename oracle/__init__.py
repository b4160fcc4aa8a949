"""CPU oracle of the KVMem hot path -- test infrastructure only.

Only the tests, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP library.
"""
from . import kvmem_oracle  # noqa: F401
