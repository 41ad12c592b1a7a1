"""CPU oracle of the SeKV decode path: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package.  The HIP library and its Python binding never do.
"""
from .sekv_oracle import *  # noqa: F401,F403
