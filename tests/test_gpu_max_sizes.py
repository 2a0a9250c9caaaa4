"""GPU parity at the widest rows the library takes (bf16 d = 16384 and float32
d = 8192: four 16-byte vectors per lane) and at three vectors per lane (bf16
d = 10000, float32 d = 5000), for every kernel family: the aggregation in each
of its source-bound instances, plain and fused with the partial update, and
over more than 9 sources; the two-phase pair; the backward (the general
kernel, the last-source kernel, with dL/dw formed or left to the caller, the
block pass with its dL/dw contraction and the partial sums' dL/dw pass).
These are the instances the other tests, at d <= 8192 bf16, do not reach.  A
few tokens keep the oracle fast."""

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import synth
from oracle import attnres_oracle as orc
from tests.gpu_util import compare, device, host, note, oracle_aggregate, same_bits, weighted_abs
from tests.test_gpu_backward import C_BWD, bounds, check, inputs

pytestmark = pytest.mark.gpu

WIDE = [("bf16", 16384), ("bf16", 10000), ("f32", 8192), ("f32", 5000)]
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("dtype,d", WIDE)
@pytest.mark.parametrize("S", [1, 2, 4, 5, 9])
def test_wide_aggregate(dtype, d, S):
    T = 7
    note(f"wide aggregate {dtype} d={d} S={S} T={T}")
    dev = device()
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=S + d, dtype=dtype, device=dev)
    w = synth.query(d, seed=d, device=dev)
    out, a = B.aggregate(H, w)
    torch.cuda.synchronize()
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(host(out), host(a), r_ref, a_ref, dtype == "bf16", f"wide aggregate {dtype} d={d} S={S}")


@pytest.mark.parametrize("dtype,d", WIDE)
@pytest.mark.parametrize("S", [10, 94])
def test_wide_many_sources(dtype, d, S):
    """More than 9 sources (Full AttnRes: batches of 9 merged by online softmax)."""
    T = 3
    note(f"wide many sources {dtype} d={d} S={S} T={T}")
    dev = device()
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=S + d, dtype=dtype, device=dev)
    w = synth.query(d, seed=S, device=dev)
    out, a = B.aggregate(H, w)
    torch.cuda.synchronize()
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(host(out), host(a), r_ref, a_ref, dtype == "bf16", f"wide many sources {dtype} d={d} S={S}")


@pytest.mark.parametrize("dtype,d", WIDE)
@pytest.mark.parametrize("n_done,partial_valid,finalize", [(0, True, False), (2, True, True), (7, True, False),
                                                           (3, False, False)])
def test_wide_fused_update(dtype, d, n_done, partial_valid, finalize):
    """Fused update + aggregation: bit-identical to the separate pair, and the
    aggregation over the updated store within the parity bar."""
    T = 5
    note(f"wide fused {dtype} d={d} n_done={n_done} partial={partial_valid} finalize={finalize}")
    dev = device()
    stores = [B.SourceStore(T, d, s_max=9, dtype=TDT[dtype], device=dev) for _ in range(2)]
    init = synth.sources(9, T, d, scale=(0.5, 50.0), seed=d + n_done, dtype=dtype, device=dev)
    for st in stores:
        st.slots.copy_(init)
        st.set_state(n_done, partial_valid)
    F = synth.layer_output(T, d, std=1.0, seed=d, tag=3, device=dev, dtype=dtype)
    w = synth.query(d, seed=n_done, device=dev)
    out_f, a_f = stores[0].accumulate_aggregate(F, finalize, w)
    stores[1].accumulate(F, finalize_block=finalize)
    out_p, a_p = stores[1].aggregate(w)
    torch.cuda.synchronize()
    assert torch.equal(stores[0].slots, stores[1].slots), "store rows differ from the separate update"
    assert torch.equal(out_f, out_p) and torch.equal(a_f, a_p), "fused result differs from the pair"
    r_ref, a_ref = oracle_aggregate(host(stores[1].sources()), host(w))
    compare(host(out_f), host(a_f), r_ref, a_ref, dtype == "bf16", f"wide fused {dtype} d={d}")


@pytest.mark.parametrize("d", [16384, 10000])
@pytest.mark.parametrize("n_completed,close", [(2, True), (6, True), (4, False)])
def test_wide_two_phase(d, n_completed, close):
    """The inter-block pass for four queries (closing the open block by
    addition where asked), then one merge, against the plain aggregation."""
    T, Bq = 6, 4
    note(f"wide two-phase d={d} n_completed={n_completed} close={close}")
    dev = device()
    st = B.SourceStore(T, d, dtype=torch.bfloat16, device=dev)
    synth.sources(9, T, d, scale=(0.5, 50.0), seed=d + n_completed, out=st.slots)
    st.set_state(n_completed, close)
    before = host(st.slots)
    F = synth.layer_output(T, d, std=1.0, seed=d, tag=5, device=dev)
    K = 1 + n_completed + (1 if close else 0)
    W = torch.stack([synth.query(d, seed=b, device=dev, tag=70 + b) for b in range(Bq)])
    inter = torch.empty((Bq, T, d), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((Bq, T, K), dtype=torch.float32, device=dev)
    st.block_prepare(F if close else None, close, B.split_queries(W), inter, logits)
    torch.cuda.synchronize()
    H = before[:K].copy()
    if close:
        H[K - 1] = orc.accumulate(before[K - 1], host(F), "bf16")
        assert same_bits(st.slots[K - 1], H[K - 1]), "closed block representation"
    for b in range(Bq):
        r_ref, a_ref = oracle_aggregate(H, host(W[b]))
        a_gpu = torch.softmax(logits[b].double(), dim=1).cpu().numpy()
        compare(host(inter[b]), a_gpu, r_ref, a_ref, True, f"wide prepare query {b}")
    F2 = synth.layer_output(T, d, std=0.3, seed=d, tag=6, device=dev)
    out, wts = st.block_merge(F2, W[1], inter[1], logits[1])
    torch.cuda.synchronize()
    partial = orc.accumulate(None, host(F2), "bf16")
    assert same_bits(st.slots[K], partial), "partial after the merge's copy"
    Hi = np.concatenate([H, partial[None]], axis=0)
    r_ref, a_ref = oracle_aggregate(Hi, host(W[1]))
    compare(host(out), host(wts), r_ref, a_ref, True, "wide merge", extra_rounding=weighted_abs(Hi, a_ref, K))


@pytest.mark.parametrize("dtype,d", WIDE)
@pytest.mark.parametrize("S,acc", [(3, 0b101), (9, 0x1FF)])
@pytest.mark.parametrize("form_dw", [True, False], ids=["dw", "coef"])
def test_wide_backward(dtype, d, S, acc, form_dw):
    """The general backward kernel (every source's row written or added); with
    dL/dw left to the caller, dL/dw summed on the host from the coefficients
    it writes for every source."""
    T = 6
    note(f"wide backward {dtype} d={d} S={S} acc={acc:#x} form_dw={form_dw}")
    H, w, g = inputs(S, T, d, TDT[dtype], seed=S + d)
    dev = H.device
    prefill = torch.randn((S, T, d), generator=torch.Generator(device=dev).manual_seed(3), device=dev)
    grads = prefill.clone()
    hand = torch.empty((T, d), dtype=TDT[dtype], device=dev)
    coef = torch.full((T, 3 * S), float("nan"), dtype=torch.float32, device=dev)
    kw = {} if form_dw else dict(form_dw=False, coef=coef, coef_stride=3 * S)
    dw = B.aggregate_backward(H, w, g, grads, accumulate=acc, grad_last=hand, **kw)
    torch.cuda.synchronize()
    if not form_dw:
        cf = host(coef).astype(np.float64).reshape(T, S, 3)
        dw = sum(cf[:, s, 1] @ host(H[s]).astype(np.float64) for s in range(S))
    pre = np.stack([host(prefill[s]) if (acc >> s) & 1 else np.zeros((T, d)) for s in range(S)])
    check(host(grads), host(dw) if form_dw else dw, host(H), host(w), host(g), f"wide backward {dtype} d={d} S={S}",
          prefill=pre)
    assert torch.equal(hand, grads[S - 1].to(TDT[dtype])), "handed-out gradient is not the row's rounding"


@pytest.mark.parametrize("dtype,d", WIDE)
@pytest.mark.parametrize("S", [1, 4, 9])
def test_wide_last_source_backward(dtype, d, S):
    """Every source but the last deferred (the streaming kernel): coefficients
    recombine to the oracle's gradients, the last row is added, dL/dw is the
    last source's share."""
    T = 6
    defer = (1 << (S - 1)) - 1
    note(f"wide last-source backward {dtype} d={d} S={S}")
    H, w, g = inputs(S, T, d, TDT[dtype], seed=3 * S + d)
    dev = H.device
    prefill = torch.randn((S, T, d), generator=torch.Generator(device=dev).manual_seed(8), device=dev)
    grads = prefill.clone()
    coef = torch.full((T, 3 * S), float("nan"), dtype=torch.float32, device=dev)
    dw = B.aggregate_backward(H, w, g, grads, accumulate=1 << (S - 1), defer=defer, coef=coef, coef_stride=3 * S)
    torch.cuda.synchronize()
    Hh, wh, gh = host(H), host(w), host(g)
    dH_ref, _, dw_src = orc.depth_attention_backward(Hh, wh, gh, per_source=True)
    bH, bw = bounds(Hh, wh, gh)
    cf = host(coef).astype(np.float64).reshape(T, S, 3)
    tiny = np.finfo(np.float32).tiny
    for s in range(S):
        if (defer >> s) & 1:
            assert torch.equal(grads[s], prefill[s]), f"deferred row {s} was written"
            rec = cf[:, s, 0:1] * gh + cf[:, s, 1:2] * wh[None] - cf[:, s, 2:3] * Hh[s]
        else:
            rec = host(grads[s]) - host(prefill[s])
        lim = C_BWD * bH[s] + 2.0 ** -22 * (np.abs(dH_ref[s]) + np.abs(host(prefill[s]))) + tiny
        assert np.all(np.abs(rec - dH_ref[s]) <= lim), f"source {s}: ratio {np.max(np.abs(rec - dH_ref[s]) / lim):.3g}"
    limw = C_BWD * bw + 2.0 ** -23 * np.abs(dw_src[S - 1]) + tiny
    assert np.all(np.abs(host(dw).astype(np.float64) - dw_src[S - 1]) <= limw), "dw share of the last source"


@pytest.mark.parametrize("dtype,d", WIDE)
def test_wide_block_backward(dtype, d):
    """The block pass over n = 3 inter-block sources and 3 layers: gradient rows
    and each layer's full dL/dw against the oracle."""
    n, Bl, T = 3, 3, 5
    note(f"wide block backward {dtype} d={d}")
    H, _, _ = inputs(n, T, d, TDT[dtype], seed=d + 1)
    dev = H.device
    Ws = [synth.query(d, seed=d, device=dev, tag=l) for l in range(Bl)]
    Gs = [synth.layer_output(T, d, std=1.0, seed=d, tag=80 + l, device=dev, dtype=dtype) for l in range(Bl)]
    prefill = torch.randn((n, T, d), generator=torch.Generator(device=dev).manual_seed(9), device=dev)
    grads = prefill.clone()
    coef = torch.empty((T, Bl, n, 3), dtype=torch.float32, device=dev)
    scratch = torch.zeros((n, T, d), dtype=torch.float32, device=dev)
    dws = [B.aggregate_backward(H, Ws[l], Gs[l], scratch, defer=(1 << n) - 1, coef=coef.view(-1)[3 * n * l:],
                                coef_stride=3 * n * Bl) for l in range(Bl)]
    B.block_backward(H, Gs, Ws, coef, grads, dws, accumulate=(1 << n) - 1)
    torch.cuda.synchronize()
    Hh = host(H)
    ref = host(prefill).astype(np.float64)
    bH_tot = np.zeros_like(ref)
    for l in range(Bl):
        dH, dw_ref = orc.depth_attention_backward(Hh, host(Ws[l]), host(Gs[l]))
        bH, bw = bounds(Hh, host(Ws[l]), host(Gs[l]))
        ref += dH
        bH_tot += bH
        e = np.abs(host(dws[l]).astype(np.float64) - dw_ref)
        assert np.all(e <= C_BWD * bw + 2.0 ** -23 * np.abs(dw_ref)), f"dL/dw layer {l}"
    err = np.abs(host(grads) - ref)
    lim = C_BWD * bH_tot + 2.0 ** -22 * np.abs(ref) + 2.0 ** -23 * np.abs(host(prefill))
    assert np.all(err <= lim), f"gradient rows: ratio {np.max(err / lim):.3g}"


@pytest.mark.parametrize("dtype,d", WIDE)
def test_wide_block_with_dw_per_block(dtype, d):
    """The schedule's deferred form at the widest rows: n = 3 inter-block
    sources and 3 layers, each with a partial sum of its own as last source;
    the layers form no dL/dw (one workgroup per token) and write n + 1 triples
    per token, attnres_partial_dw forms the partials' share and the block pass
    (at that wider coefficient stride) adds the rest: each partial's gradient
    row, the inter-block rows and every layer's whole dL/dw against the oracle."""
    n, Bl, T = 3, 3, 5
    m = 3 * (n + 1)
    note(f"wide block with dL/dw per block {dtype} d={d}")
    H, _, _ = inputs(n, T, d, TDT[dtype], seed=d + 2)
    dev = H.device
    Ws = [synth.query(d, seed=d, device=dev, tag=10 + l) for l in range(Bl)]
    Gs = [synth.layer_output(T, d, std=1.0, seed=d, tag=90 + l, device=dev, dtype=dtype) for l in range(Bl)]
    Ps = [synth.layer_output(T, d, std=3.0, seed=d, tag=95 + l, device=dev, dtype=dtype) for l in range(Bl)]
    prefill = torch.randn((n, T, d), generator=torch.Generator(device=dev).manual_seed(10), device=dev)
    grads = prefill.clone()
    coef = torch.full((T, Bl, n + 1, 3), float("nan"), dtype=torch.float32, device=dev)
    own = [torch.zeros((n + 1, T, d), dtype=torch.float32, device=dev) for _ in range(Bl)]
    for l in range(Bl):
        B.aggregate_backward(H, Ws[l], Gs[l], own[l], last_source=Ps[l], defer=(1 << n) - 1,
                             coef=coef.view(-1)[m * l:], coef_stride=m * Bl, form_dw=False)
    dws = [torch.full((d,), float("nan"), dtype=torch.float32, device=dev) for _ in range(Bl)]
    B.partial_dw(Ps, coef.view(-1)[3 * n + 1:], m * Bl, m, dws)
    B.block_backward(H, Gs, Ws, coef, grads, dws, accumulate=(1 << n) - 1, coef_layer_stride=m)
    torch.cuda.synchronize()
    Hh = host(H)
    ref = host(prefill).astype(np.float64)
    bH_tot = np.zeros_like(ref)
    tiny = np.finfo(np.float32).tiny
    for l in range(Bl):
        src = np.concatenate([Hh, host(Ps[l])[None]])
        dH, dw_ref = orc.depth_attention_backward(src, host(Ws[l]), host(Gs[l]))
        bH, bw = bounds(src, host(Ws[l]), host(Gs[l]))
        ref += dH[:n]
        bH_tot += bH[:n]
        e = np.abs(host(own[l][n]) - dH[n])
        assert np.all(e <= C_BWD * bH[n] + 2.0 ** -22 * np.abs(dH[n]) + tiny), f"partial row of layer {l}"
        e = np.abs(host(dws[l]).astype(np.float64) - dw_ref)
        assert np.all(e <= C_BWD * bw + 2.0 ** -23 * np.abs(dw_ref) + tiny), f"dL/dw layer {l}"
    err = np.abs(host(grads) - ref)
    lim = C_BWD * bH_tot + 2.0 ** -22 * np.abs(ref) + 2.0 ** -23 * np.abs(host(prefill))
    assert np.all(err <= lim), f"gradient rows: ratio {np.max(err / lim):.3g}"
