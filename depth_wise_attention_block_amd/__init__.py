"""Block Attention-Residuals depth aggregation on MI355X (gfx950).

The compute path is ``libattnres.so`` (hand-written HIP kernels behind a C ABI,
``include/attnres.h``); :mod:`.binding` marshals torch device tensors into it.
The library is loaded on first use and a missing or unloadable library raises
``RuntimeError``: there is no fallback implementation.
"""

__all__ = ["synth"]
