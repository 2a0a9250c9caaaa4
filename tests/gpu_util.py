"""Shared helpers of the GPU parity tests: device checks, host copies, and the
comparison of GPU results with the oracle at the stated tolerances."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

from oracle import attnres_oracle as orc

# Tolerances of the parity bar.
BF16_WEIGHT_ATOL = 1e-3        # depth weights, bf16 sources
BF16_OUT_RTOL_OF_MAX = 1e-2    # |dr| <= 1e-2 * max|r|, bf16 output
F32_OUT_RTOL_OF_MAX = 1e-5     # fp32 mode: max|dr| / max|r| <= 1e-5
F32_WEIGHT_ATOL = 1e-5
# Tighter element-wise bound for bf16 outputs: one rounding to bf16 (half an ulp,
# 2^-8 relative) plus float32 accumulation error.
BF16_OUT_ELEMENT_REL = 2.0 ** -8
BF16_OUT_ELEMENT_ABS_OF_MAX = 1e-4


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def note(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Exact host copy as float32 (bf16 widens exactly) or float32."""
    return t.detach().float().cpu().numpy()


def oracle_aggregate(H: np.ndarray, w: np.ndarray, chunk: int = 256):
    """Oracle over token chunks (bounded float64 temporaries)."""
    S, T, d = H.shape
    r = np.empty((T, d), np.float64)
    a = np.empty((T, S), np.float64)
    for t0 in range(0, T, chunk):
        r[t0:t0 + chunk], a[t0:t0 + chunk] = orc.depth_attention(H[:, t0:t0 + chunk], w)
    return r, a


def weighted_abs(H: np.ndarray, a: np.ndarray, upto: int) -> np.ndarray:
    """sum_{s < upto} a_s |H_s| per element: the size of a weighted sum's terms,
    the scale of one extra bf16 rounding of a partial weighted sum."""
    H = np.asarray(H, np.float64)
    return sum(a[:, s:s + 1] * np.abs(H[s]) for s in range(upto))


def compare(r_gpu: np.ndarray, a_gpu, r_ref: np.ndarray, a_ref: np.ndarray, bf16: bool, what: str,
            extra_rounding=None):
    """Assert the parity bar; returns the observed errors.  ``extra_rounding``
    (bf16 only): per-element magnitude of an intermediate result that the path
    stored in bf16 (e.g. the two-phase schedule's inter-block rows); it widens
    the element-wise bound by one bf16 rounding of that magnitude."""
    r_gpu = np.asarray(r_gpu, np.float64)
    rmax = float(np.max(np.abs(r_ref))) if r_ref.size else 0.0
    dr = np.abs(r_gpu - r_ref)
    err_r = float(dr.max()) if dr.size else 0.0
    err_a = 0.0
    if a_gpu is not None and a_ref.size:
        err_a = float(np.max(np.abs(np.asarray(a_gpu, np.float64) - a_ref)))
    assert np.all(np.isfinite(r_gpu)), f"{what}: non-finite output"
    if bf16:
        assert err_a <= BF16_WEIGHT_ATOL, f"{what}: weight error {err_a:.3e}"
        assert err_r <= BF16_OUT_RTOL_OF_MAX * rmax, f"{what}: output error {err_r:.3e} vs max {rmax:.3e}"
        bound = BF16_OUT_ELEMENT_REL * np.abs(r_ref) + BF16_OUT_ELEMENT_ABS_OF_MAX * rmax
        if extra_rounding is not None:
            bound = bound + BF16_OUT_ELEMENT_REL * np.asarray(extra_rounding, np.float64)
        worst = np.unravel_index(np.argmax(dr - bound), dr.shape) if dr.size else None
        assert np.all(dr <= bound), f"{what}: element {worst} off by {dr[worst]:.3e} > {bound[worst]:.3e}"
    else:
        assert err_a <= F32_WEIGHT_ATOL, f"{what}: weight error {err_a:.3e}"
        assert err_r <= F32_OUT_RTOL_OF_MAX * rmax, f"{what}: output error {err_r:.3e} vs max {rmax:.3e}"
    note(f"{what}: max|dr|={err_r:.3e} (max|r|={rmax:.3e}) max|da|={err_a:.3e}")
    return err_r, err_a


def same_bits(x: torch.Tensor, y: np.ndarray) -> bool:
    """Bitwise equality of a GPU tensor with float32 values in numpy."""
    hx = host(x).view(np.uint32)
    return np.array_equal(hx, np.asarray(y, np.float32).view(np.uint32))
