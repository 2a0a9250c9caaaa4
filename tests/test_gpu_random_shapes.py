"""Seeded random shapes through the hot path against the oracle: the
aggregation over strided sources, the fused update + aggregation (bit-exact
against the pair of separate calls and within the parity bar of the oracle),
and the aggregation backward with random accumulate / defer masks, with dL/dw
formed or left to the caller; and the partial sums' dL/dw pass at random layer
counts, strides and missing rows.  Every case prints its parameters before it
runs."""

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import synth
from oracle import attnres_oracle as orc
from tests.gpu_util import compare, device, host, note, oracle_aggregate
from tests.test_gpu_backward import C_BWD, bounds

pytestmark = pytest.mark.gpu


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        vec = 8 if dtype == "bf16" else 4
        d = int(vec * rng.integers(1, (8192 if dtype == "bf16" else 4096) // vec + 1))
        if rng.random() < 0.3:
            d = 7168
        S = int(rng.integers(1, 10))
        T = int(rng.integers(0, 200))
        pad = int(vec * rng.integers(0, 64)) if rng.random() < 0.5 else 0
        out.append((k, dtype, S, T, d, pad, int(rng.integers(0, 2 ** 31))))
    return out


def _sources(S, T, d, pad, dtype, seed, dev):
    """S rows of [T, d] at a row stride of T*d + pad (pad = 0: contiguous)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    base = torch.empty(S * (T * d + pad) + 16, dtype=tdt, device=dev)
    H = base[: S * (T * d + pad)].view(S, T * d + pad)[:, : T * d].view(S, T, d) if S * T * d else \
        torch.empty((S, T, d), dtype=tdt, device=dev)
    if S * T * d:
        H.copy_(synth.sources(S, T, d, scale=(0.2, 30.0), seed=seed, dtype=dtype, device=dev))
    return H


@pytest.mark.parametrize("case", _cases(48, 2024), ids=lambda c: f"{c[1]}-S{c[2]}-T{c[3]}-d{c[4]}-pad{c[5]}")
def test_random_aggregate(case):
    k, dtype, S, T, d, pad, seed = case
    note(f"random aggregate #{k}: {dtype} S={S} T={T} d={d} pad={pad}")
    dev = device()
    H = _sources(S, T, d, pad, dtype, seed, dev)
    w = synth.query(d, seed=seed, device=dev)
    out, a = B.aggregate(H, w)
    torch.cuda.synchronize()
    if T == 0:
        return
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(host(out), host(a), r_ref, a_ref, dtype == "bf16", f"random #{k}")


@pytest.mark.parametrize("case", _cases(32, 77), ids=lambda c: f"{c[1]}-S{c[2]}-T{c[3]}-d{c[4]}")
def test_random_fused_update(case):
    k, dtype, S, T, d, _, seed = case
    dev = device()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(seed)
    # a store state with room for the update: n_done completed blocks (<= 7),
    # an open partial or not (its first layer: the update is a copy), closing or not
    n_done = min(S - 1, 7)
    partial_valid = bool(rng.random() < 0.7)
    finalize = bool(rng.random() < 0.3)
    note(f"random fused #{k}: {dtype} T={T} d={d} n_done={n_done} partial={partial_valid} finalize={finalize}")
    stores = [B.SourceStore(T, d, s_max=9, dtype=tdt, device=dev) for _ in range(2)]
    init = synth.sources(9, T, d, scale=(0.2, 30.0), seed=seed, dtype=dtype, device=dev)
    for st in stores:
        st.slots.copy_(init)
        st.set_state(n_done, partial_valid)
    F = synth.layer_output(T, d, std=1.0, seed=seed, tag=3, device=dev, dtype=dtype)
    w = synth.query(d, seed=seed, device=dev)
    out_f, a_f = stores[0].accumulate_aggregate(F, finalize, w)
    stores[1].accumulate(F, finalize_block=finalize)
    out_p, a_p = stores[1].aggregate(w)
    torch.cuda.synchronize()
    assert torch.equal(stores[0].slots, stores[1].slots), "store rows differ from the separate update"
    assert torch.equal(out_f, out_p) and torch.equal(a_f, a_p), "fused result differs from the pair"
    if T:
        H = host(stores[1].sources())
        r_ref, a_ref = oracle_aggregate(H, host(w))
        compare(host(out_f), host(a_f), r_ref, a_ref, dtype == "bf16", f"random fused #{k}")


@pytest.mark.parametrize("case", _cases(24, 99), ids=lambda c: f"{c[1]}-S{c[2]}-T{c[3]}-d{c[4]}")
def test_random_backward(case):
    k, dtype, S, T, d, pad, seed = case
    rng = np.random.default_rng(seed)
    acc = int(rng.integers(0, 2 ** S))
    defer = int(rng.integers(0, 2 ** S)) if rng.random() < 0.5 else 0
    note(f"random backward #{k}: {dtype} S={S} T={T} d={d} pad={pad} acc={acc:#x} defer={defer:#x}")
    dev = device()
    H = _sources(S, T, d, pad, dtype, seed, dev)
    w = synth.query(d, seed=seed, device=dev)
    g = synth.layer_output(T, d, std=1.0, seed=seed, tag=4, device=dev, dtype=dtype)
    prefill = torch.randn((S, T, d), generator=torch.Generator(device=dev).manual_seed(seed % 1000), device=dev)
    grads = prefill.clone()
    coef = torch.zeros((max(T, 1), 3 * S), dtype=torch.float32, device=dev)
    dw = B.aggregate_backward(H, w, g, grads, accumulate=acc, defer=defer, coef=coef if defer else None,
                              coef_stride=3 * S)
    torch.cuda.synchronize()
    if T == 0:
        assert not dw.any()
        return
    Hh, wh, gh = host(H), host(w), host(g)
    dH_ref, _, dw_src = orc.depth_attention_backward(Hh, wh, gh, per_source=True)
    bH, bw = bounds(Hh, wh, gh)
    got, cf = host(grads), host(coef).astype(np.float64).reshape(T, S, 3)
    tiny = np.finfo(np.float32).tiny
    for s in range(S):
        if (defer >> s) & 1:
            assert torch.equal(grads[s], prefill[s]), f"deferred row {s} written"
            rec = cf[:, s, 0:1] * gh + cf[:, s, 1:2] * wh[None] - cf[:, s, 2:3] * Hh[s]
        else:
            rec = got[s] - (host(prefill[s]) if (acc >> s) & 1 else 0.0)
        lim = C_BWD * bH[s] + 2.0 ** -22 * (np.abs(dH_ref[s]) + np.abs(host(prefill[s]))) + tiny
        assert np.all(np.abs(rec - dH_ref[s]) <= lim), f"source {s}: ratio {np.max(np.abs(rec - dH_ref[s]) / lim):.3g}"
    share = sum((dw_src[s] for s in range(S) if not (defer >> s) & 1), np.zeros(d))
    limw = C_BWD * bw + 2.0 ** -23 * np.abs(share) + tiny
    assert np.all(np.abs(host(dw).astype(np.float64) - share) <= limw), "dw share"


@pytest.mark.parametrize("case", _cases(16, 515), ids=lambda c: f"{c[1]}-S{c[2]}-T{c[3]}-d{c[4]}")
def test_random_backward_without_dw(case):
    """grad_w NULL: every source's coefficients written; they recombine to the
    oracle's dH_s for every source, the non-deferred rows match the oracle, and
    sum_t sum_s c1 H_s (on the host) is the oracle's whole dL/dw."""
    k, dtype, S, T, d, pad, seed = case
    rng = np.random.default_rng(seed)
    acc = int(rng.integers(0, 2 ** S))
    defer = int(rng.integers(0, 2 ** S)) if rng.random() < 0.5 else 0
    note(f"random backward without dw #{k}: {dtype} S={S} T={T} d={d} pad={pad} acc={acc:#x} defer={defer:#x}")
    dev = device()
    H = _sources(S, T, d, pad, dtype, seed, dev)
    w = synth.query(d, seed=seed, device=dev)
    g = synth.layer_output(T, d, std=1.0, seed=seed, tag=5, device=dev, dtype=dtype)
    prefill = torch.randn((S, T, d), generator=torch.Generator(device=dev).manual_seed(seed % 997), device=dev)
    grads = prefill.clone()
    cs = 3 * S + int(rng.integers(0, 4))
    coef = torch.full((max(T, 1) * cs,), float("nan"), dtype=torch.float32, device=dev)
    assert B.aggregate_backward(H, w, g, grads, accumulate=acc, defer=defer, coef=coef, coef_stride=cs,
                                form_dw=False) is None
    torch.cuda.synchronize()
    if T == 0:
        assert torch.equal(grads, prefill)
        return
    Hh, wh, gh = host(H), host(w), host(g)
    dH_ref, dw_ref = orc.depth_attention_backward(Hh, wh, gh)
    bH, bw = bounds(Hh, wh, gh)
    got = host(grads)
    cf = host(coef).astype(np.float64)[: T * cs].reshape(T, cs)[:, : 3 * S].reshape(T, S, 3)
    assert not np.any(np.isnan(cf)), "a source's coefficients were not written"
    tiny = np.finfo(np.float32).tiny
    for s in range(S):
        lim = C_BWD * bH[s] + 2.0 ** -22 * (np.abs(dH_ref[s]) + np.abs(host(prefill[s]))) + tiny
        rec = cf[:, s, 0:1] * gh + cf[:, s, 1:2] * wh[None] - cf[:, s, 2:3] * Hh[s]
        assert np.all(np.abs(rec - dH_ref[s]) <= lim), f"coefficients of source {s}"
        if (defer >> s) & 1:
            assert torch.equal(grads[s], prefill[s]), f"deferred row {s} written"
        else:
            row = got[s] - (host(prefill[s]) if (acc >> s) & 1 else 0.0)
            assert np.all(np.abs(row - dH_ref[s]) <= lim), f"row {s}"
    dw = sum(cf[:, s, 1] @ Hh[s].astype(np.float64) for s in range(S))
    limw = C_BWD * bw + 2.0 ** -23 * np.abs(dw_ref) + tiny
    assert np.all(np.abs(dw - dw_ref) <= limw), "dL/dw from the coefficients"


def _pdw_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        vec = 8 if dtype == "bf16" else 4
        d = int(vec * rng.integers(1, (8192 if dtype == "bf16" else 4096) // vec + 1))
        out.append((k, dtype, int(rng.integers(1, 17)), int(rng.integers(0, 3000)), d, int(rng.integers(0, 2 ** 31))))
    return out


@pytest.mark.parametrize("case", _pdw_cases(16, 616), ids=lambda c: f"{c[1]}-B{c[2]}-T{c[3]}-d{c[4]}")
def test_random_partial_dw(case):
    """attnres_partial_dw at random layer counts, coefficient strides and
    missing rows, against a float64 sum; rows without data are zeroed."""
    k, dtype, Bl, T, d, seed = case
    rng = np.random.default_rng(seed)
    dev = device()
    present = [bool(rng.random() < 0.75) for _ in range(Bl)]
    cls = int(rng.integers(1, 6))
    cs = Bl * cls + int(rng.integers(0, 5))
    off = int(rng.integers(0, 4))
    note(f"random partial dw #{k}: {dtype} B={Bl} T={T} d={d} rows={present} cls={cls} cs={cs} off={off}")
    rows = [synth.layer_output(T, d, std=2.0, seed=seed, tag=20 + l, device=dev, dtype=dtype) if present[l] else None
            for l in range(Bl)]
    coef = torch.randn((max(T, 1) * cs + off + 1,), generator=torch.Generator(device=dev).manual_seed(seed % 991),
                       device=dev)
    dws = [torch.full((d,), float("nan"), dtype=torch.float32, device=dev) for _ in range(Bl)]
    B.partial_dw(rows, coef[off:], cs, cls, dws)
    torch.cuda.synchronize()
    c = host(coef).astype(np.float64)[off:]
    for l in range(Bl):
        got = host(dws[l]).astype(np.float64)
        if rows[l] is None or T == 0:
            assert np.all(got == 0.0), f"layer {l}: no row, yet not zero"
            continue
        X = host(rows[l]).astype(np.float64)
        cl = c[np.arange(T) * cs + l * cls]
        want, mag = cl @ X, np.abs(cl) @ np.abs(X)
        assert np.all(np.abs(got - want) <= 1e-4 * mag + 1e-30), f"layer {l}"
