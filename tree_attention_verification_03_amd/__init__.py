"""MI355X-native verification hot path of EAGLE-2-style dynamic-tree speculative decoding.

The computation lives in ``libspectree.so`` (hand-written HIP kernels for
gfx950 behind the C ABI of ``include/spec_tree.h``); this package is its thin
Python binding. The library is loaded on first use and its absence raises -
there is no fallback implementation.
"""
from . import ops  # noqa: F401
from ._lib import LIB_PATH, SpecError, load  # noqa: F401

__all__ = ["ops", "load", "LIB_PATH", "SpecError"]
