"""Optional roctx ranges around the depth schedule's steps.

With ``ATTNRES_ROCTX=1`` in the environment the ROCm roctx library is loaded
through ctypes and the schedule drivers push one named range per step (a
layer's aggregation, a block's inter-block pass, partial sums and gradient-row
pass, the output layer), which ``rocprofv3 --marker-trace`` records next to the
kernels.  The ranges are host-side: they bracket the enqueueing of a step's
launches.  Without the variable (or without the library) every ``span`` is the
same no-op context and nothing is loaded.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

_NULL = contextlib.nullcontext()
_LIB_NAMES = ("librocprofiler-sdk-roctx.so.1", "libroctx64.so.4")


def _load():
    if os.environ.get("ATTNRES_ROCTX") != "1":
        return None
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    for name in _LIB_NAMES:
        for path in (os.path.join(rocm, "lib", name), name):
            try:
                lib = ctypes.CDLL(path)
            except OSError:
                continue
            lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
            lib.roctxRangePushA.restype = ctypes.c_int
            lib.roctxRangePop.argtypes = []
            lib.roctxRangePop.restype = ctypes.c_int
            return lib
    return None


_lib = _load()
ENABLED = _lib is not None


@contextlib.contextmanager
def _range(name: str):
    _lib.roctxRangePushA(name.encode())
    try:
        yield
    finally:
        _lib.roctxRangePop()


def span(kind: str, index: int | None = None):
    """A context that marks one schedule step, e.g. ``span("layer", 7)``."""
    if _lib is None:
        return _NULL
    return _range(kind if index is None else f"{kind} {index}")
