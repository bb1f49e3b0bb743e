"""fp64 CPU oracle for the ring-attention rank share.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and
by bench.py's cpu_baseline leg, never by the product library or its binding.
"""
from .ref import *  # noqa: F401,F403
from . import ref  # noqa: F401
