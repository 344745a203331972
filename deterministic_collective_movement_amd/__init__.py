"""deterministic_collective_movement_amd -- rank-ordered gather (rog) for MI355X.

The library is the C-ABI shared object ``librog.so`` (declared in
``include/rog.h``) built from the hand-written HIP kernels under ``csrc/``.
``deterministic_collective_movement_amd.rog`` is the thin ctypes binding with
the same entry-point names.  Attributes of the binding are reachable from the
package itself (``dcm.rog_gather``); the library is loaded on first use.
"""

__all__ = ["rog", "workloads"]


def __getattr__(name):
    if name.startswith("rog_") or name in ("RogError", "ROG_PATH_AUTO", "ROG_PATH_SINGLE_WG",
                                           "ROG_PATH_MULTI_WG", "library_path"):
        from . import rog as _rog
        return getattr(_rog, name)
    raise AttributeError(name)
