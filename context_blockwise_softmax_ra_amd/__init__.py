"""MI355X-native ring-attention rank share: HIP kernels behind a C ABI (libra.so).

``_lib`` binds the C entry points under their own names; ``ring`` runs the
simulated ranks of a context-parallel group in turn on one GPU.
"""
from ._lib import *  # noqa: F401,F403
from . import _lib  # noqa: F401

__all__ = [n for n in dir(_lib) if n.startswith("ra_") or n.isupper()]
