"""ctypes binding of libattnres.so: argument marshalling only.

Every entry point mirrors a C function of ``include/attnres.h`` and passes torch
device pointers, sizes and the current HIP stream straight through.  All
arithmetic happens in the library's HIP kernels; a missing library raises
``RuntimeError`` -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# ATTNRES_LIBRARY names another build of the same ABI (the CPU tests point it at
# the sanitized host-only build); by default the HIP library next to this file
LIB_PATH = os.environ.get("ATTNRES_LIBRARY") or os.path.join(HERE, "libattnres.so")

BF16, F32 = 0, 1
MAX_SOURCES = 9            # Block AttnRes store slots
MAX_SOURCES_FULL = 256     # one aggregation (Full AttnRes / sublayer granularity)
MAX_INTER_SOURCES = 8      # two-phase: inter-block sources per pass
MAX_BLOCK_QUERIES = 16     # two-phase: layer queries per pass
MAX_D_BF16, MAX_D_F32 = 16384, 8192   # widest rows (ATTNRES_MAX_D_BF16 / _F32)
STATIC_SCRATCH_BYTES = 16 << 20       # ATTNRES_STATIC_SCRATCH_BYTES
OK, EINVAL, EUNSUPPORTED, EALIAS, ELAUNCH, ESTATE = 0, -1, -2, -3, -4, -5
_DTYPE_CODE = {torch.bfloat16: BF16, torch.float32: F32}


class AttnResError(RuntimeError):
    """A libattnres call returned a negative status."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func}: {strerror(status)} (status {status})")


class attnres_store_t(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("T", ctypes.c_int64), ("slot_stride", ctypes.c_int64),
                ("d", ctypes.c_int32), ("s_max", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_completed", ctypes.c_int32), ("partial_valid", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class attnres_launch_t(ctypes.Structure):
    _fields_ = [("threads", ctypes.c_int32), ("vecs_per_lane", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("tokens_per_group", ctypes.c_int32), ("xcd_run", ctypes.c_int32)]


_SIGNATURES = {
    "attnres_version": (ctypes.c_int, []),
    "attnres_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "attnres_aggregate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]),
    "attnres_store_init": (ctypes.c_int, [ctypes.POINTER(attnres_store_t), ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]),
    "attnres_store_sources": (ctypes.c_int, [ctypes.POINTER(attnres_store_t)]),
    "attnres_accumulate": (ctypes.c_int, [ctypes.POINTER(attnres_store_t), ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p]),
    "attnres_accumulate_aggregate": (ctypes.c_int, [ctypes.POINTER(attnres_store_t), ctypes.c_void_p, ctypes.c_int32,
                                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                                    ctypes.c_void_p]),
    "attnres_block_prepare": (ctypes.c_int, [ctypes.POINTER(attnres_store_t), ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]),
    "attnres_block_merge": (ctypes.c_int, [ctypes.POINTER(attnres_store_t), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_float, ctypes.c_void_p]),
    "attnres_split_queries": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "attnres_add_rows": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "attnres_aggregate_backward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p,
                                                  ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int32,
                                                  ctypes.c_void_p]),
    "attnres_aggregate_backward_static": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                         ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                         ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint32,
                                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                         ctypes.c_void_p, ctypes.c_float, ctypes.c_int32,
                                                         ctypes.c_void_p]),
    "attnres_partial_sums": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_void_p]),
    "attnres_block_backward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                              ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p,
                                              ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_int32, ctypes.c_void_p]),
    "attnres_partial_dw": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_void_p]),
    "attnres_partial_dw_workspace": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]),
    "attnres_block_backward_workspace": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                        ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]),
    "attnres_aggregate_backward_workspace": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                            ctypes.POINTER(ctypes.c_int64)]),
    "attnres_aggregate_config": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.POINTER(attnres_launch_t)]),
}

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises RuntimeError if it is not built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                       "`python -m depth_wise_attention_block_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def strerror(status: int) -> str:
    return lib().attnres_strerror(int(status)).decode()


def version() -> int:
    return int(lib().attnres_version())


def _check(func: str, status: int) -> int:
    if status < 0:
        raise AttnResError(func, status)
    return status


def _stream(device: torch.device, stream) -> int:
    """The stream handle for a launch on ``device``, which must be a GPU: the C
    ABI takes plain pointers and cannot tell host memory from device memory."""
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, not {device}")
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(getattr(stream, "cuda_stream", stream))


def _same_gpu(dev: torch.device, *named) -> None:
    """Every tensor argument of a launch must sit on the launch's GPU ``dev``:
    the C ABI takes plain pointers, so a host tensor (or one on another GPU)
    among device tensors would reach a kernel as a foreign address.  ``named``
    holds ``(name, tensor-or-None)`` pairs; lists of tensors are checked item
    by item."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, not {dev}")
    for name, t in named:
        items = t if isinstance(t, (list, tuple)) else (t,)
        for i, x in enumerate(items):
            if x is not None and x.device != dev:
                label = f"{name}[{i}]" if isinstance(t, (list, tuple)) else name
                raise ValueError(f"{label} must be on {dev}, the GPU of this launch, not on {x.device}")


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPE_CODE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32") from None


def aggregate_config(S: int, T: int, d: int, dtype=torch.bfloat16, num_cus: int = 256) -> dict:
    """Launch shape the library picks (host-side query, no GPU needed)."""
    cfg = attnres_launch_t()
    _check("attnres_aggregate_config",
           lib().attnres_aggregate_config(S, T, d, _DTYPE_CODE[dtype], num_cus, ctypes.byref(cfg)))
    return {"threads": cfg.threads, "vecs_per_lane": cfg.vecs_per_lane, "grid": cfg.grid,
            "tokens_per_group": cfg.tokens_per_group, "xcd_run": cfg.xcd_run}


def aggregate(sources: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None,
              weights: torch.Tensor | None = None, *, want_weights: bool = True, eps: float = 1e-5,
              stream=None):
    """``attnres_aggregate`` on ``sources`` ``[S, T, d]`` (rows contiguous; any
    source stride), query ``w`` ``[d]`` float32.  Returns ``(out, weights)``;
    ``weights`` is ``None`` when not wanted."""
    if sources.dim() != 3:
        raise ValueError("sources must be [S, T, d]")
    S, T, d = sources.shape
    if T > 0 and (sources.stride(2) != 1 or sources.stride(1) != d):
        raise ValueError("each source must be a contiguous [T, d] block")
    dev = sources.device
    _same_gpu(dev, ("w", w), ("out", out), ("weights", weights))
    if out is None:
        out = torch.empty((T, d), dtype=sources.dtype, device=dev)
    if weights is None and want_weights:
        weights = torch.empty((T, S), dtype=torch.float32, device=dev)
    for name, t in (("w", w), ("out", out)) + ((("weights", weights),) if weights is not None else ()):
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    if w.dtype != torch.float32 or w.numel() != d:
        raise ValueError("w must be float32 with d elements")
    if out.dtype != sources.dtype or out.numel() != T * d:
        raise ValueError("out must match the sources' dtype and hold T*d elements")
    if weights is not None and (weights.dtype != torch.float32 or weights.numel() != T * S):
        raise ValueError("weights must be float32 with T*S elements")
    stride = sources.stride(0) if S > 1 else T * d
    rc = lib().attnres_aggregate(sources.data_ptr(), S, T, d, stride, w.data_ptr(), out.data_ptr(),
                                 weights.data_ptr() if weights is not None else None, float(eps),
                                 _dtype_code(sources), _stream(dev, stream))
    _check("attnres_aggregate", rc)
    return out, weights


def backward_workspace_bytes(T: int, d: int, dtype=torch.bfloat16) -> int:
    """``attnres_aggregate_backward_workspace`` on the current device."""
    out = ctypes.c_int64()
    _check("attnres_aggregate_backward_workspace",
           lib().attnres_aggregate_backward_workspace(T, d, _DTYPE_CODE[dtype], ctypes.byref(out)))
    return out.value


def block_workspace_bytes(T: int, d: int, B: int, dtype=torch.bfloat16) -> int:
    """``attnres_block_backward_workspace`` on the current device."""
    out = ctypes.c_int64()
    _check("attnres_block_backward_workspace",
           lib().attnres_block_backward_workspace(T, d, B, _DTYPE_CODE[dtype], ctypes.byref(out)))
    return out.value


def add_rows(a: torch.Tensor | None, b: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """``attnres_add_rows``: ``out = a + b`` as the partial-sum update forms it
    (``out = b`` when ``a`` is None); rows ``[T, d]``, contiguous."""
    T, d = b.shape
    _same_gpu(b.device, ("a", a), ("out", out))
    for name, t in (("b", b), ("out", out)) + ((("a", a),) if a is not None else ()):
        if not t.is_contiguous() or t.dtype != b.dtype or tuple(t.shape) != (T, d) or t.device != b.device:
            raise ValueError(f"{name} must be a contiguous [T, d] tensor like b")
    _check("attnres_add_rows", lib().attnres_add_rows(a.data_ptr() if a is not None else None, b.data_ptr(),
                                                      out.data_ptr(), T, d, _dtype_code(b), _stream(b.device, stream)))
    return out


def aggregate_backward(sources: torch.Tensor, w: torch.Tensor, grad_out: torch.Tensor, grad_sources: torch.Tensor,
                       *, last_source: torch.Tensor | None = None, accumulate=0, defer=0,
                       coef: torch.Tensor | None = None, coef_stride: int = 0, grad_w: torch.Tensor | None = None,
                       grad_last: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                       form_dw: bool = True, eps: float = 1e-5, stream=None) -> torch.Tensor | None:
    """``attnres_aggregate_backward``: writes (or, for the sources whose bit is
    set in the ``accumulate`` mask, adds) dL/dH into ``grad_sources``
    ``[S, T, d]`` float32 (rows contiguous, any row stride) and returns dL/dw
    (``grad_w``, float32 ``[d]``).  ``sources`` holds the S rows, or the first
    S-1 when ``last_source`` ``[T, d]`` gives the last one apart.  ``grad_out``
    is dL/dr ``[T, d]`` in the sources' dtype; ``grad_last`` (optional,
    ``[T, d]`` sources' dtype) receives the new gradient of the last source.
    Sources in the ``defer`` mask keep their gradient rows untouched and write
    their coefficients to ``coef`` (float32, ``coef_stride`` floats per token,
    may be a view starting mid-row) for :func:`block_backward`, which also adds
    their share of dL/dw: the returned ``grad_w`` sums the other sources only.
    With ``form_dw=False`` no dL/dw is formed (``grad_w`` must be None; the C
    call gets NULL): every source's coefficients go to ``coef``, for
    :func:`block_backward` and :func:`partial_dw`, and None is returned."""
    if grad_sources.dim() != 3 or sources.dim() != 3:
        raise ValueError("sources and grad_sources must be 3-D")
    S, T, d = grad_sources.shape
    if sources.shape[0] != (S - 1 if last_source is not None else S) or tuple(sources.shape[1:]) != (T, d):
        raise ValueError("sources must hold S rows (S-1 with last_source) of [T, d]")
    for name, t in (("sources", sources), ("grad_sources", grad_sources)):
        if T > 0 and t.shape[0] > 0 and (t.stride(2) != 1 or t.stride(1) != d):
            raise ValueError(f"each row of {name} must be a contiguous [T, d] block")
    if last_source is not None and (not last_source.is_contiguous() or last_source.dtype != sources.dtype
                                    or last_source.numel() != T * d):
        raise ValueError("last_source must be a contiguous [T, d] tensor like the sources")
    dev = grad_sources.device
    _same_gpu(dev, ("sources", sources), ("last_source", last_source), ("w", w), ("grad_out", grad_out),
              ("coef", coef), ("grad_w", grad_w), ("grad_last", grad_last), ("workspace", workspace))
    if grad_sources.dtype != torch.float32:
        raise ValueError("grad_sources must be float32")
    if not form_dw and grad_w is not None:
        raise ValueError("form_dw=False takes no grad_w")
    if form_dw and grad_w is None:
        grad_w = torch.empty(d, dtype=torch.float32, device=dev)
    if form_dw and workspace is None:
        nbytes = backward_workspace_bytes(T, d, sources.dtype)
        workspace = torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device=dev)
    checks = (("w", w, torch.float32, d), ("grad_out", grad_out, sources.dtype, T * d))
    if form_dw:
        checks += (("grad_w", grad_w, torch.float32, d),)
    if grad_last is not None:
        checks += (("grad_last", grad_last, sources.dtype, T * d),)
    for name, t, dt, n in checks:
        if t.device != dev or not t.is_contiguous() or t.dtype != dt or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous {dt} tensor with {n} elements on {dev}")
    if workspace is not None and (not workspace.is_contiguous() or workspace.device != dev):
        raise ValueError("workspace must be a contiguous device tensor")
    mask = accumulate if isinstance(accumulate, int) else sum(1 << i for i, a in enumerate(accumulate) if a)
    if (defer or not form_dw) and (coef is None or coef.dtype != torch.float32 or coef.device != dev):
        raise ValueError("deferred sources (and form_dw=False) need a float32 coef buffer on the device")
    if (defer or not form_dw) and T > 0:
        # the kernel writes (T - 1) * coef_stride + 3 S floats from coef's first element at most
        top = S if not form_dw else (defer & ((1 << S) - 1)).bit_length()
        need = (T - 1) * int(coef_stride) + 3 * top
        if not coef.is_contiguous() or coef.numel() < need:
            raise ValueError(f"coef must be a contiguous float32 tensor of at least {need} elements")
    src_stride = sources.stride(0) if sources.shape[0] > 1 else T * d
    grad_stride = grad_sources.stride(0) if S > 1 else T * d
    src_ptr = sources.data_ptr() if sources.shape[0] > 0 else None
    rc = lib().attnres_aggregate_backward(
        src_ptr, S, T, d, src_stride, last_source.data_ptr() if last_source is not None else None, w.data_ptr(),
        grad_out.data_ptr(), grad_sources.data_ptr(),
        grad_stride, mask & 0xFFFFFFFF, defer & 0xFFFFFFFF, coef.data_ptr() if (defer or not form_dw) else None,
        int(coef_stride), grad_last.data_ptr() if grad_last is not None else None,
        grad_w.data_ptr() if form_dw else None, workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0, float(eps),
        _dtype_code(sources), _stream(dev, stream))
    _check("attnres_aggregate_backward", rc)
    return grad_w


def partial_sums(layer_outs, out: torch.Tensor, stream=None) -> torch.Tensor:
    """``attnres_partial_sums``: ``out[k]`` = F_0 + ... + F_k as the store forms
    them; ``layer_outs`` is a list of ``[T, d]`` tensors, ``out`` ``[count, T, d]``
    (rows contiguous, any row stride)."""
    count = len(layer_outs)
    if count == 0 or out.dim() != 3 or out.shape[0] < count:
        raise ValueError("out must be [>= count, T, d]")
    _, T, d = out.shape
    _same_gpu(out.device, ("layer_outs", list(layer_outs)))
    for F in layer_outs:
        if F.dtype != out.dtype or not F.is_contiguous() or tuple(F.shape) != (T, d):
            raise ValueError("each layer output must be a contiguous [T, d] tensor like out")
    if T > 0 and (out.stride(2) != 1 or out.stride(1) != d):
        raise ValueError("each row of out must be a contiguous [T, d] block")
    arr = (ctypes.c_void_p * count)(*[F.data_ptr() for F in layer_outs])
    _check("attnres_partial_sums", lib().attnres_partial_sums(arr, count, T, d, out.data_ptr(),
                                                              out.stride(0) if count > 1 else T * d,
                                                              _dtype_code(out), _stream(out.device, stream)))
    return out


def block_backward(sources: torch.Tensor, grad_outs, queries, coef: torch.Tensor, grad_sources: torch.Tensor,
                   grad_ws, *, accumulate=0, grad_last: torch.Tensor | None = None, coef_layer_stride: int = 0,
                   workspace: torch.Tensor | None = None, stream=None) -> None:
    """``attnres_block_backward``: add the B layers' deferred contributions into
    the n inter-block gradient rows ``grad_sources`` ``[n, T, d]`` float32, and
    the deferred sources' share of each layer's dL/dw into ``grad_ws[l]``
    (float32 ``[d]``).  ``sources`` ``[n, T, d]``; ``grad_outs`` / ``queries``:
    B tensors ``[T, d]`` / ``[d]``; ``coef`` contiguous float32 with
    ``T * B * m`` elements, ``[T, B, m]``, layer l's n triples first in its m
    floats, m = ``coef_layer_stride`` (0: m = 3n, ``[T, B, n, 3]``)."""
    n, T, d = grad_sources.shape
    Bl = len(grad_outs)
    if sources.shape != grad_sources.shape or len(queries) != Bl or len(grad_ws) != Bl:
        raise ValueError("sources must match grad_sources; one query and one dL/dw row per upstream gradient")
    dev = grad_sources.device
    _same_gpu(dev, ("sources", sources), ("grad_outs", list(grad_outs)), ("queries", list(queries)),
              ("coef", coef), ("grad_ws", list(grad_ws)), ("grad_last", grad_last), ("workspace", workspace))
    for name, t in (("sources", sources), ("grad_sources", grad_sources)):
        if T > 0 and (t.stride(2) != 1 or t.stride(1) != d):
            raise ValueError(f"each row of {name} must be a contiguous [T, d] block")
    m = coef_layer_stride or 3 * n
    if coef.dtype != torch.float32 or not coef.is_contiguous() or coef.numel() != T * Bl * m:
        raise ValueError(f"coef must be a contiguous float32 tensor of T * B * {m} elements")
    for g in grad_outs:
        if g.dtype != sources.dtype or not g.is_contiguous() or g.numel() != T * d:
            raise ValueError("each upstream gradient must be a contiguous [T, d] tensor like the sources")
    for name, rows in (("query", queries), ("dL/dw row", grad_ws)):
        for w in rows:
            if w.dtype != torch.float32 or not w.is_contiguous() or w.numel() != d or w.device != dev:
                raise ValueError(f"each {name} must be a contiguous float32 [d] tensor on {dev}")
    if workspace is None:
        nbytes = block_workspace_bytes(T, d, Bl, sources.dtype)
        workspace = torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device=dev)
    if not workspace.is_contiguous() or workspace.device != dev:
        raise ValueError("workspace must be a contiguous device tensor")
    garr = (ctypes.c_void_p * Bl)(*[g.data_ptr() for g in grad_outs])
    warr = (ctypes.c_void_p * Bl)(*[w.data_ptr() for w in queries])
    dwarr = (ctypes.c_void_p * Bl)(*[w.data_ptr() for w in grad_ws])
    mask = accumulate if isinstance(accumulate, int) else sum(1 << i for i, a in enumerate(accumulate) if a)
    _check("attnres_block_backward", lib().attnres_block_backward(
        sources.data_ptr(), n, T, d, sources.stride(0) if n > 1 else T * d, Bl, garr, warr, coef.data_ptr(),
        int(coef_layer_stride), grad_sources.data_ptr(), grad_sources.stride(0) if n > 1 else T * d, mask & 0xFFFFFFFF,
        grad_last.data_ptr() if grad_last is not None else None, dwarr, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _dtype_code(sources), _stream(dev, stream)))


def partial_dw_workspace_bytes(T: int, d: int, B: int, dtype=torch.bfloat16) -> int:
    """``attnres_partial_dw_workspace`` on the current device."""
    out = ctypes.c_int64(0)
    _check("attnres_partial_dw_workspace",
           lib().attnres_partial_dw_workspace(T, d, B, _DTYPE_CODE[dtype], ctypes.byref(out)))
    return int(out.value)


def partial_dw(rows, coef: torch.Tensor | None, coef_stride: int, coef_layer_stride: int, grad_ws, *,
               workspace: torch.Tensor | None = None, stream=None) -> None:
    """``attnres_partial_dw``: ``grad_ws[l]`` (float32 ``[d]``) is overwritten
    with the sum over tokens t of ``coef[t * coef_stride + l * coef_layer_stride]
    * rows[l][t]``; ``rows`` are B tensors ``[T, d]`` (or None: that layer's row
    is zeroed); ``coef`` a float32 device tensor whose first element is layer
    0's coefficient for token 0 (a view may start mid-row)."""
    Bl = len(grad_ws)
    if len(rows) != Bl or Bl == 0:
        raise ValueError("one row (or None) per dL/dw row")
    d = grad_ws[0].numel()
    given = [r for r in rows if r is not None]
    dev = grad_ws[0].device
    _same_gpu(dev, ("rows", given), ("coef", coef), ("grad_ws", list(grad_ws)), ("workspace", workspace))
    T = given[0].shape[0] if given else 0
    dt = given[0].dtype if given else torch.float32
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}; use bfloat16 or float32")
    for r in given:
        if r.dtype != dt or not r.is_contiguous() or tuple(r.shape) != (T, d):
            raise ValueError("each row must be a contiguous [T, d] tensor, all of one dtype")
    for w in grad_ws:
        if w.dtype != torch.float32 or not w.is_contiguous() or w.numel() != d:
            raise ValueError(f"each dL/dw row must be a contiguous float32 [d] tensor on {dev}")
    if given and T > 0:
        if coef is None or coef.dtype != torch.float32 or not coef.is_contiguous():
            raise ValueError("rows need a contiguous float32 coef tensor")
        # the last layer's coefficient of the last token, counted from coef's first element
        need = (T - 1) * int(coef_stride) + (Bl - 1) * int(coef_layer_stride) + 1
        if coef.numel() < need:
            raise ValueError(f"coef must hold at least {need} elements")
    if workspace is None:
        nbytes = partial_dw_workspace_bytes(T, d, Bl, dt)
        workspace = torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device=dev)
    if not workspace.is_contiguous() or workspace.device != dev:
        raise ValueError("workspace must be a contiguous device tensor")
    rarr = (ctypes.c_void_p * Bl)(*[r.data_ptr() if r is not None else None for r in rows])
    dwarr = (ctypes.c_void_p * Bl)(*[w.data_ptr() for w in grad_ws])
    _check("attnres_partial_dw", lib().attnres_partial_dw(
        rarr, Bl, T, d, coef.data_ptr() if coef is not None else None, int(coef_stride), int(coef_layer_stride),
        dwarr, workspace.data_ptr(), workspace.numel() * workspace.element_size(), _DTYPE_CODE[dt],
        _stream(dev, stream)))


def prepared_query_shape(n: int, d: int):
    """Shape of :func:`split_queries`' output for n queries of width d:
    ``[ceil(n/4), 2, d/8, 4, 8]`` bf16 -- group, plane (hi, lo), 8-element chunk,
    query within the group, element."""
    return ((n + 3) // 4, 2, d // 8, 4, 8)


def split_queries(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """``attnres_split_queries``: float32 queries ``[n, d]`` -> the prepared
    bf16 form ``prepared_query_shape(n, d)`` (hi and lo halves, queries grouped
    by four) that the two-phase pass reads."""
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 [n, d] tensor")
    n, d = w.shape
    _same_gpu(w.device, ("out", out))
    shape = prepared_query_shape(n, d)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=w.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != shape or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 {list(shape)} tensor")
    _check("attnres_split_queries", lib().attnres_split_queries(w.data_ptr(), n, d, out.data_ptr(),
                                                                _stream(w.device, stream)))
    return out


def unpack_prepared_queries(ws: torch.Tensor, n: int) -> torch.Tensor:
    """Inverse layout of :func:`split_queries` (no arithmetic): ``[n, 2, d]``
    with plane 0 = hi, plane 1 = lo."""
    G, P, C, four, eight = ws.shape
    rows = ws.permute(0, 3, 1, 2, 4).reshape(G * four, P, C * eight)
    return rows[:n]


class SourceStore:
    """Device slots ``[s_max, T, d]`` plus the C store bookkeeping.

    Slot 0 is h_0 (fill ``store.h0``); completed block representations and the
    running partial sum follow.  ``sources()`` is the live ``[S, T, d]`` view the
    next aggregation reads.
    """

    def __init__(self, T: int, d: int, *, s_max: int = MAX_SOURCES, dtype=torch.bfloat16,
                 device="cuda", slots: torch.Tensor | None = None):
        if slots is None:
            slots = torch.empty((s_max, T, d), dtype=dtype, device=device)
        if slots.shape != (s_max, T, d) or not slots.is_contiguous():
            raise ValueError("slots must be a contiguous [s_max, T, d] tensor")
        self.slots = slots
        self.T, self.d, self.s_max = T, d, s_max
        self._st = attnres_store_t()
        _check("attnres_store_init",
               lib().attnres_store_init(ctypes.byref(self._st), slots.data_ptr(), s_max, T, d, 0,
                                        _dtype_code(slots)))

    @property
    def h0(self) -> torch.Tensor:
        return self.slots[0]

    @property
    def n_completed(self) -> int:
        return self._st.n_completed

    @property
    def partial_valid(self) -> bool:
        return bool(self._st.partial_valid)

    def num_sources(self) -> int:
        return _check("attnres_store_sources", lib().attnres_store_sources(ctypes.byref(self._st)))

    def sources(self) -> torch.Tensor:
        return self.slots[: self.num_sources()]

    def reset(self) -> None:
        """Forget every block (h_0 stays)."""
        self.set_state(0, False)

    def set_state(self, n_completed: int, partial_valid: bool) -> None:
        """Declare which slots hold data (for slots filled directly, e.g. with
        synthetic block representations); checked by the library."""
        old = (self._st.n_completed, self._st.partial_valid)
        self._st.n_completed, self._st.partial_valid = int(n_completed), int(bool(partial_valid))
        try:
            _check("attnres_store_sources", lib().attnres_store_sources(ctypes.byref(self._st)))
        except AttnResError:
            self._st.n_completed, self._st.partial_valid = old
            raise

    def accumulate(self, layer_out: torch.Tensor, finalize_block: bool = False, stream=None) -> None:
        _same_gpu(self.slots.device, ("layer_out", layer_out))
        if layer_out.dtype != self.slots.dtype or layer_out.device != self.slots.device \
                or not layer_out.is_contiguous() or layer_out.numel() != self.T * self.d:
            raise ValueError("layer_out must be a contiguous [T, d] tensor like the store")
        rc = lib().attnres_accumulate(ctypes.byref(self._st), layer_out.data_ptr(), int(bool(finalize_block)),
                                      _stream(self.slots.device, stream))
        _check("attnres_accumulate", rc)

    def aggregate(self, w: torch.Tensor, out=None, weights=None, *, want_weights=True, eps=1e-5, stream=None):
        return aggregate(self.sources(), w, out, weights, want_weights=want_weights, eps=eps, stream=stream)

    def accumulate_aggregate(self, layer_out: torch.Tensor, finalize_block: bool, w: torch.Tensor, out=None,
                             weights=None, *, want_weights=True, eps=1e-5, stream=None):
        """``attnres_accumulate_aggregate``: add ``layer_out`` into the current
        block (closing it if asked), then aggregate the live sources with the
        next layer's query ``w`` -- one kernel.  Returns ``(out, weights)``."""
        _same_gpu(self.slots.device, ("layer_out", layer_out), ("w", w), ("out", out), ("weights", weights))
        if layer_out.dtype != self.slots.dtype or layer_out.device != self.slots.device \
                or not layer_out.is_contiguous() or layer_out.numel() != self.T * self.d:
            raise ValueError("layer_out must be a contiguous [T, d] tensor like the store")
        S = 1 + self.n_completed + (1 if finalize_block else 0) + (0 if finalize_block else 1)
        dev = self.slots.device
        if out is None:
            out = torch.empty((self.T, self.d), dtype=self.slots.dtype, device=dev)
        if weights is None and want_weights:
            weights = torch.empty((self.T, S), dtype=torch.float32, device=dev)
        if w.dtype != torch.float32 or w.numel() != self.d or w.device != dev or not w.is_contiguous():
            raise ValueError("w must be a contiguous float32 [d] tensor on the store's device")
        if out.dtype != self.slots.dtype or out.numel() != self.T * self.d or not out.is_contiguous():
            raise ValueError("out must be a contiguous [T, d] tensor of the store's dtype")
        if weights is not None and (weights.dtype != torch.float32 or weights.numel() != self.T * S
                                    or not weights.is_contiguous()):
            raise ValueError("weights must be a contiguous float32 tensor with T*S elements")
        rc = lib().attnres_accumulate_aggregate(ctypes.byref(self._st), layer_out.data_ptr(), int(bool(finalize_block)),
                                                w.data_ptr(), out.data_ptr(),
                                                weights.data_ptr() if weights is not None else None, float(eps),
                                                _stream(dev, stream))
        _check("attnres_accumulate_aggregate", rc)
        return out, weights

    # ---- two-phase schedule -------------------------------------------------

    def block_prepare(self, layer_out, close_block: bool, w_split: torch.Tensor, inter: torch.Tensor,
                      logits: torch.Tensor, weights0=None, *, eps=1e-5, stream=None):
        """``attnres_block_prepare``: optionally close the open block with
        ``layer_out``, then one pass over the K inter-block sources for the B
        queries ``w_split`` (:func:`split_queries` of the B queries).  ``inter``
        is ``[B, T, d]`` (rows may be strided along dim 0), ``logits``
        ``[B, T, K]`` float32 with ``K = 1 + n_completed`` after the close;
        ``weights0`` optional ``[T, K]``."""
        dev = self.slots.device
        _same_gpu(dev, ("layer_out", layer_out), ("w_split", w_split), ("inter", inter), ("logits", logits),
                  ("weights0", weights0))
        B = inter.shape[0] if inter.dim() == 3 else -1
        if w_split.dtype != torch.bfloat16 or tuple(w_split.shape) != prepared_query_shape(B, self.d) \
                or not w_split.is_contiguous():
            raise ValueError("w_split must be split_queries() of the B queries (contiguous bfloat16)")
        if inter.dim() != 3 or inter.shape[0] != B or inter.shape[1:] != (self.T, self.d) or \
                inter.dtype != self.slots.dtype or (self.T > 0 and (inter.stride(2) != 1 or inter.stride(1) != self.d)):
            raise ValueError("inter must be [B, T, d] of the store dtype with contiguous rows")
        K = 1 + self.n_completed + (1 if close_block else 0)
        if logits.dtype != torch.float32 or logits.numel() != B * self.T * K or not logits.is_contiguous():
            raise ValueError("logits must be a contiguous float32 tensor with B*T*K elements")
        if weights0 is not None and (weights0.dtype != torch.float32 or weights0.numel() != self.T * K
                                     or not weights0.is_contiguous()):
            raise ValueError("weights0 must be a contiguous float32 tensor with T*K elements")
        if close_block and (layer_out is None or layer_out.dtype != self.slots.dtype or
                            not layer_out.is_contiguous() or layer_out.numel() != self.T * self.d):
            raise ValueError("closing needs a contiguous [T, d] layer_out like the store")
        stride = inter.stride(0) if B > 1 else self.T * self.d
        rc = lib().attnres_block_prepare(ctypes.byref(self._st), layer_out.data_ptr() if close_block else None,
                                         int(bool(close_block)), w_split.data_ptr(), B, inter.data_ptr(), stride,
                                         logits.data_ptr(), weights0.data_ptr() if weights0 is not None else None,
                                         float(eps), _stream(dev, stream))
        _check("attnres_block_prepare", rc)

    def block_merge(self, layer_out: torch.Tensor, w: torch.Tensor, inter: torch.Tensor, logits: torch.Tensor,
                    out=None, weights=None, *, want_weights=True, eps=1e-5, stream=None):
        """``attnres_block_merge``: add ``layer_out`` into the partial and merge it
        with the inter-block part (``inter`` row ``[T, d]`` and its ``logits``
        ``[T, K]``) for this layer's query ``w``.  ``out`` may be ``inter``
        itself.  Returns ``(out, weights)``, weights ``[T, K + 1]``."""
        dev = self.slots.device
        _same_gpu(dev, ("layer_out", layer_out), ("w", w), ("inter", inter), ("logits", logits), ("out", out),
                  ("weights", weights))
        K = 1 + self.n_completed
        for name, t, dt, n in (("layer_out", layer_out, self.slots.dtype, self.T * self.d),
                               ("w", w, torch.float32, self.d), ("inter", inter, self.slots.dtype, self.T * self.d),
                               ("logits", logits, torch.float32, self.T * K)):
            if t.dtype != dt or t.numel() != n or not t.is_contiguous() or t.device != dev:
                raise ValueError(f"{name} must be a contiguous {dt} tensor with {n} elements on {dev}")
        if out is None:
            out = torch.empty((self.T, self.d), dtype=self.slots.dtype, device=dev)
        if weights is None and want_weights:
            weights = torch.empty((self.T, K + 1), dtype=torch.float32, device=dev)
        if out.dtype != self.slots.dtype or out.numel() != self.T * self.d or not out.is_contiguous():
            raise ValueError("out must be a contiguous [T, d] tensor of the store dtype")
        if weights is not None and (weights.dtype != torch.float32 or weights.numel() != self.T * (K + 1)
                                    or not weights.is_contiguous()):
            raise ValueError("weights must be a contiguous float32 tensor with T*(K+1) elements")
        rc = lib().attnres_block_merge(ctypes.byref(self._st), layer_out.data_ptr(), w.data_ptr(), inter.data_ptr(),
                                       logits.data_ptr(), out.data_ptr(),
                                       weights.data_ptr() if weights is not None else None, float(eps),
                                       _stream(dev, stream))
        _check("attnres_block_merge", rc)
        return out, weights
