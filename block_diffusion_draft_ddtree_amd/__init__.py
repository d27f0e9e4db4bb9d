"""libddtree: DDTree's per-round draft-tree hot path for AMD MI355X (gfx950).

The compute lives in ``libddtree.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/ddtree.h``). ``binding`` is a thin ctypes layer
with the same function names; it marshals torch tensors to device pointers
and the current HIP stream. ``synth`` draws the seeded synthetic inputs.
The shared library is loaded on first use and its absence is an error.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "binding"]


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(__name__ + ".binding")
    raise AttributeError(name)
