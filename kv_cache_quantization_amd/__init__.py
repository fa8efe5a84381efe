"""KIVI KV-cache quantization and decode attention for AMD MI355X (gfx950).

The computation lives in ``libkivi.so`` (hand-written HIP kernels behind the C
ABI of ``include/kivi.h``); this package marshals arguments to it.

* ``kivi``   -- ctypes binding, one function per C entry point.
* ``cache``  -- ``KiviCache``: a torch-allocated device buffer bound to a cache.
* ``synth``  -- seeded synthetic K/V/q generators (no KIVI arithmetic).
* ``build``  -- compiles ``libkivi.so`` in-tree with hipcc for gfx950.
"""
from .kivi import KiviError  # noqa: F401

__all__ = ["KiviError", "KiviCache"]


def __getattr__(name):
    if name == "KiviCache":
        from .cache import KiviCache
        return KiviCache
    raise AttributeError(name)
