"""deterministic_collective_movement_amd -- rank-ordered gather and rank-ordered
sum (rog) for MI355X.

The library is the C-ABI shared object ``librog.so`` (declared in
``include/rog.h``) built from the hand-written HIP kernels under ``csrc/``.
``deterministic_collective_movement_amd.rog`` is the thin ctypes binding with
the same entry-point names.  Attributes of the binding are reachable from the
package itself (``dcm.rog_gather``); the library is loaded on first use.
"""
import importlib

__all__ = ["rog", "workloads", "build"]


def __getattr__(name):
    if name.startswith("__") or name in ("rog", "workloads", "build"):
        raise AttributeError(name)
    mod = importlib.import_module(__name__ + ".rog")
    try:
        return getattr(mod, name)
    except AttributeError:
        raise AttributeError(name) from None
