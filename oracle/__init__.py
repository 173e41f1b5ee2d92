"""CPU oracle for 3D Block Sparse Attention -- test infrastructure only.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg. The product library never imports it.
"""

from .bsa_oracle import *  # noqa: F401,F403
from .bsa_oracle import __all__  # noqa: F401
