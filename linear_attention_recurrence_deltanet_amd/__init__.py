"""libgdn: Gated DeltaNet (gated delta rule) forward for AMD MI355X (gfx950).

The compute path is the C-ABI shared library ``libgdn.so`` (hand-written HIP
kernels, see ``csrc/``); ``gdn.py`` is a thin ctypes binding with the same
entry-point names.  ``inputs.py`` holds the seeded synthetic workloads.
Nothing here falls back to a CPU implementation: if the library is missing
the binding raises.
"""
__all__ = ["gdn", "inputs"]


def __getattr__(name):
    if name == "gdn":
        from . import gdn as _g
        return _g
    if name == "inputs":
        from . import inputs as _i
        return _i
    raise AttributeError(name)
