"""libcartattn: cartridge attention on MI355X (gfx950).

The compute lives in the HIP shared library ``libcartattn.so`` built from
``csrc/``; ``long_context_kv_amd.cartattn`` is its ctypes binding. Importing
this package loads nothing: import the binding module to load the library.
"""

__all__ = ["cartattn", "workloads"]
