"""libgdn: Gated DeltaNet (gated delta rule) forward for AMD MI355X (gfx950).

The compute path is the C-ABI shared library ``libgdn.so`` (hand-written HIP
kernels, see ``csrc/``); ``gdn.py`` is a thin ctypes binding with the same
entry-point names.  ``inputs.py`` holds the seeded synthetic workloads.
Nothing here falls back to a CPU implementation: if the library is missing
the binding raises.  Submodules are imported explicitly, e.g.
``from linear_attention_recurrence_deltanet_amd import gdn``.
"""
