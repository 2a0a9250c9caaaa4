"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random tensors with the shapes and value distributions
of the workloads; it holds none of the aggregation's arithmetic, so both the
HIP path and the CPU oracle may consume what it produces.

Distributions (per workload):

* sources: every source s gets one scale ``exp(U(ln lo, ln hi))`` (log-uniform),
  its entries are ``N(0, 1) * scale`` drawn in float32 and rounded to the store
  dtype;
* pseudo-queries: ``N(0, 4/d)`` in float32;
* layer outputs: ``N(0, std^2)`` rounded to the store dtype.

Each tensor gets its own ``torch.Generator`` seeded from ``(seed, tag)``, so the
values depend only on the seed, the tag, the shape and the device (CPU and GPU
generators give different streams; parity always feeds the oracle the very
values the GPU saw).
"""

from __future__ import annotations

import math

import torch

#: Workloads: the fp32 CPU-sized case, the single-layer aggregate, the decode
#: batches, the long-context prefill chunk and the 93-layer depth schedule.
WORKLOADS = {
    "fp32_small": dict(T=64, d=256, S=4, dtype="f32", scale=(0.1, 10.0)),
    "layer_t4096": dict(T=4096, d=7168, S=9, dtype="bf16", scale=(0.5, 50.0)),
    "decode": dict(T=(1, 8, 64, 256), d=7168, S=9, dtype="bf16", scale=(0.5, 50.0),
                   layer_out_std=1.0),
    "prefill_t262144": dict(T=262144, d=7168, S=9, dtype="bf16", scale=(0.5, 50.0),
                            layer_out_std=1.0),
    "schedule_93": dict(T=32768, d=7168, layers=93, block_size=12, dtype="bf16",
                        h0_scale=1.0, layer_out_std=0.1),
}

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _generator(seed: int, tag: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed((int(seed) * 1_000_003 + int(tag) * 7919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def source_scales(S: int, lo: float, hi: float, seed: int):
    """One log-uniform scale per source (CPU draw, identical on every device)."""
    g = _generator(seed, 1, "cpu")
    u = torch.rand(S, generator=g, dtype=torch.float64)
    return [math.exp(math.log(lo) + (math.log(hi) - math.log(lo)) * float(x)) for x in u]


def fill_normal_(out: torch.Tensor, std: float, seed: int, tag: int,
                 chunk_rows: int = 8192) -> torch.Tensor:
    """Fill a ``[rows, d]`` tensor with ``N(0, std^2)`` drawn in float32, rounded to
    ``out.dtype``; drawn in row chunks to bound float32 temporaries."""
    g = _generator(seed, tag, out.device)
    rows, d = out.shape
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        tmp = torch.randn((r1 - r0, d), generator=g, dtype=torch.float32, device=out.device)
        if std != 1.0:
            tmp.mul_(std)
        out[r0:r1].copy_(tmp)
    return out


def sources(S: int, T: int, d: int, *, scale=(0.5, 50.0), seed: int = 0,
            dtype: str = "bf16", device="cpu", out: torch.Tensor | None = None) -> torch.Tensor:
    """``[S, T, d]`` source-major sources, source s = N(0,1) * scale_s."""
    if out is None:
        out = torch.empty((S, T, d), dtype=_TORCH_DTYPE[dtype], device=device)
    for s, sc in enumerate(source_scales(S, scale[0], scale[1], seed)):
        fill_normal_(out[s].view(T, d), sc, seed, 100 + s)
    return out


def query(d: int, seed: int = 0, device="cpu", tag: int = 0) -> torch.Tensor:
    """Pseudo-query ``w ~ N(0, 4/d)`` in float32."""
    w = torch.empty((1, d), dtype=torch.float32, device=device)
    fill_normal_(w, 2.0 / math.sqrt(d), seed, 10_000 + tag)
    return w.view(d)


def layer_output(T: int, d: int, *, std: float, seed: int = 0, tag: int = 0,
                 dtype: str = "bf16", device="cpu", out: torch.Tensor | None = None) -> torch.Tensor:
    """One layer's output ``F_l ~ N(0, std^2)`` as ``[T, d]``."""
    if out is None:
        out = torch.empty((T, d), dtype=_TORCH_DTYPE[dtype], device=device)
    return fill_normal_(out, std, seed, 20_000 + tag)


def token_sample(T: int, count: int, edge: int, seed: int = 0) -> torch.Tensor:
    """Sorted unique token indices: ``edge`` first, ``edge`` last and ``count``
    random ones -- the rows checked one by one at sizes the oracle cannot cover."""
    g = _generator(seed, 3, "cpu")
    parts = [torch.arange(0, min(edge, T)), torch.arange(max(0, T - edge), T),
             torch.randint(0, max(T, 1), (count,), generator=g)]
    return torch.unique(torch.cat(parts)) if T > 0 else torch.zeros(0, dtype=torch.long)
