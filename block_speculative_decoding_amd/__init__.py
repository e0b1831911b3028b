"""MI355X-native block-parallel speculative draft-and-verify step.

The work is done by ``libdfspec.so`` (hand-written HIP for gfx950, C ABI in
``include/dfspec.h``); :mod:`.dfspec` is its thin ctypes binding.  Importing
the binding requires the built library and raises otherwise — there is no
fallback path.
"""
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdfspec.so")


def binding():
    """Import and return the ctypes binding (raises ImportError if the library is missing)."""
    from . import dfspec
    return dfspec
