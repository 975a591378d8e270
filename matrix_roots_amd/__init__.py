"""MI355X-native EMA-Gram quarter-power preconditioner step.

The compute path is the C-ABI library ``libmatrix_roots.so`` (hand-written
HIP kernels for gfx950) declared in ``include/matrix_roots.h``; this package
is a thin ctypes binding over it.  The library is loaded on first use, and a
missing library raises instead of falling back to anything else.
"""

from __future__ import annotations

__all__ = [
    "gram_ema_update",
    "inv_quarter_root_batched",
    "precondition_apply",
    "library",
]


def __getattr__(name):
    if name in __all__:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
