"""fp64 CPU oracle — test infrastructure only (see te_oracle's header).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the HIP library and its Python binding never do.
"""
from .te_oracle import *  # noqa: F401,F403
from .te_oracle import rel_l2  # noqa: F401
