"""Reference ("oracle") implementation of Reduced Matrix Multiplication.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the cpu_baseline leg of bench.py.  The GPU library never imports it.
"""
from .oracle import *  # noqa: F401,F403
