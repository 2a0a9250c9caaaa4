"""GPU parity of the backward pass: attnres_aggregate_backward against the
oracle's depth_attention_backward, its exact properties, the row update used to
recompute partial sums, and the reverse-order Block AttnRes schedule against
the oracle's run_schedule_backward.

Tolerance (float32 results against the float64 oracle on the same inputs).  The
kernel forms u_s = g . H_s, the sums of squares and w . H_s in float32 over d
products, w as bf16 hi + lo (2^-17 relative), then delta_s = a_s (u_s - ubar).
The error of delta_s is therefore relative to M_s = a_s (|u|_s + sum a |u|),
with |u|_s = sum_j |g_j H_s,j|, not to delta_s itself (it is a difference).
Element-wise:
    |d dH_s[j]| <= c (a_s |g_j| + (M_s / rho_s)(|w_j| + |z_s| |k_s[j]| / d))
    |d dw[j]|   <= c sum_{t,s} (M_s / rho_s) |H_s[j]|
with c = 2e-4: float32 accumulation over d = 7168 products is ~sqrt(d) 2^-24 ~
5e-6 relative in the typical case (d 2^-24 = 4e-4 at worst), the hi + lo query
~8e-6; c leaves an order of magnitude above the typical case.
"""

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import schedule, synth
from oracle import attnres_oracle as orc
from tests.gpu_util import device, host, note

pytestmark = pytest.mark.gpu

C_BWD = 2e-4


def bounds(H, w, g, eps=orc.EPS):
    """Magnitude bounds of dH [S,T,d] and dw [d] (see the module docstring)."""
    H = np.asarray(H, np.float64)
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    S, T, d = H.shape
    rms = np.sqrt(np.mean(H * H, -1, keepdims=True) + eps)            # [S,T,1]
    keys = H / rms
    z = (keys @ w).T                                                   # [T,S]
    a = orc.softmax(z, axis=1)
    U = np.stack([np.sum(np.abs(g * H[s]), axis=1) for s in range(S)], axis=1)   # [T,S]
    M = a * (U + np.sum(a * U, axis=1, keepdims=True))                 # [T,S]
    coef = (M.T[:, :, None] / rms)                                     # [S,T,1]
    bH = a.T[:, :, None] * np.abs(g)[None] + coef * (np.abs(w)[None, None] + np.abs(z.T)[:, :, None] * np.abs(keys) / d)
    bw = np.sum(coef * np.abs(H), axis=(0, 1))
    return bH, bw


def check(dH_gpu, dw_gpu, H, w, g, what, prefill=None):
    """dH (and dw unless dw_gpu is None) against the oracle within the bounds."""
    dH_ref, dw_ref = orc.depth_attention_backward(H, w, g)
    if prefill is not None:
        dH_ref = dH_ref + prefill
    bH, bw = bounds(H, w, g)
    errH = np.abs(np.asarray(dH_gpu, np.float64) - dH_ref)
    # float32 rounding of a result (and of prefill + result) is within the bound's slack; below
    # float32's smallest normal a result cannot be carried at all (one-hot weights leave terms of
    # 1e-115 in float64 that are 0 in float32)
    limH = C_BWD * bH + 2.0 ** -23 * np.abs(dH_ref) + np.finfo(np.float32).tiny
    rH = float(np.max(errH / limH))
    rw = 0.0
    if dw_gpu is not None:
        errw = np.abs(np.asarray(dw_gpu, np.float64) - dw_ref)
        limw = C_BWD * bw + 2.0 ** -23 * np.abs(dw_ref) + np.finfo(np.float32).tiny
        rw = float(np.max(errw / limw))
    note(f"{what}: max err / bound dH {rH:.3g} dw {rw:.3g}")
    assert rH <= 1.0, f"{what}: dH error {np.max(errH):.3e} exceeds the bound (ratio {rH:.3g})"
    assert rw <= 1.0, f"{what}: dw error exceeds the bound (ratio {rw:.3g})"


def inputs(S, T, d, dtype, seed):
    dev = device()
    scale = (0.5, 50.0) if dtype == torch.bfloat16 else (0.1, 10.0)
    name = "bf16" if dtype == torch.bfloat16 else "f32"
    H = synth.sources(S, T, d, scale=scale, seed=seed, device=dev, dtype=name)
    w = synth.query(d, seed=seed, device=dev)
    g = synth.layer_output(T, d, std=1.0, seed=seed, tag=77, device=dev, dtype=name)
    return H, w, g


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("S", [1, 2, 5, 9])
@pytest.mark.parametrize("T,d", [(37, 7168), (5, 264), (300, 7176), (64, 256)])
def test_backward_matches_oracle(dtype, S, T, d):
    note(f"backward dtype={dtype} S={S} T={T} d={d}")
    H, w, g = inputs(S, T, d, dtype, seed=S * 100 + T)
    dev = H.device
    # every other source accumulates into a random float32 prefill
    mask = sum(1 << s for s in range(S) if s % 2 == 1)
    prefill = torch.randn((S, T, d), generator=torch.Generator(device=dev).manual_seed(3), device=dev)
    grads = prefill.clone()
    dw = B.aggregate_backward(H, w, g, grads, accumulate=mask)
    torch.cuda.synchronize()
    pre = host(prefill)
    for s in range(S):
        if not (mask >> s) & 1:
            pre[s] = 0.0
    check(host(grads), host(dw), host(H), host(w), host(g), f"S={S} T={T} d={d}", prefill=pre)


def test_backward_accumulate_is_one_float32_addition():
    H, w, g = inputs(6, 33, 1032, torch.bfloat16, seed=5)
    dev = H.device
    fresh = torch.empty((6, 33, 1032), dtype=torch.float32, device=dev)
    B.aggregate_backward(H, w, g, fresh)
    prefill = torch.randn(fresh.shape, generator=torch.Generator(device=dev).manual_seed(9), device=dev)
    acc = prefill.clone()
    B.aggregate_backward(H, w, g, acc, accumulate=(1 << 6) - 1)
    torch.cuda.synchronize()
    assert torch.equal(acc, prefill + fresh)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_backward_grad_last_is_the_rounded_last_row(dtype):
    H, w, g = inputs(4, 41, 520, dtype, seed=6)
    dev = H.device
    grads = torch.randn((4, 41, 520), generator=torch.Generator(device=dev).manual_seed(2), device=dev)
    last = torch.empty((41, 520), dtype=dtype, device=dev)
    B.aggregate_backward(H, w, g, grads, accumulate=0b1010, grad_last=last)
    torch.cuda.synchronize()
    assert torch.equal(last, grads[3].to(dtype))          # torch's conversion rounds to nearest even


def test_backward_is_bitwise_deterministic():
    H, w, g = inputs(9, 700, 7168, torch.bfloat16, seed=7)
    dev = H.device
    outs = []
    for _ in range(2):
        grads = torch.empty((9, 700, 7168), dtype=torch.float32, device=dev)
        dw = B.aggregate_backward(H, w, g, grads)
        outs.append((grads, dw))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_deferred_backward_and_block_pass_are_bitwise_deterministic():
    """The streaming kernel (every source but the last deferred) and the block
    pass with its dL/dw contraction give bit-identical results run to run."""
    n, Bl, T, d = 6, 5, 300, 7168
    H, _, _ = inputs(n + 1, T, d, torch.bfloat16, seed=17)
    dev = H.device
    Ws = [synth.query(d, seed=17, device=dev, tag=l) for l in range(Bl)]
    Gs = [synth.layer_output(T, d, std=1.0, seed=17, tag=90 + l, device=dev) for l in range(Bl)]
    runs = []
    for _ in range(2):
        grads = torch.zeros((n + 1, T, d), dtype=torch.float32, device=dev)
        coef = torch.empty((T, Bl, n, 3), dtype=torch.float32, device=dev)
        dws = [B.aggregate_backward(H, Ws[l], Gs[l], grads, accumulate=1 << n, defer=(1 << n) - 1,
                                    coef=coef.view(-1)[3 * n * l:], coef_stride=3 * n * Bl) for l in range(Bl)]
        B.block_backward(H[:n], Gs, Ws, coef, grads[:n], dws)
        runs.append((grads, coef, dws))
    torch.cuda.synchronize()
    (g0, c0, w0), (g1, c1, w1) = runs
    assert torch.equal(g0, g1) and torch.equal(c0, c1)
    assert all(torch.equal(a, b) for a, b in zip(w0, w1))


def test_backward_workspace_too_small_is_rejected():
    """Both backward entry points check the workspace size against the launch
    they would make and launch nothing when it is short."""
    n, Bl, T, d = 3, 2, 64, 1024
    H, w, g = inputs(n, T, d, torch.bfloat16, seed=18)
    dev = H.device
    grads = torch.zeros((n, T, d), dtype=torch.float32, device=dev)
    need = B.backward_workspace_bytes(T, d)
    short = torch.empty(max(need // 4 - 4, 4), dtype=torch.float32, device=dev)
    with pytest.raises(B.AttnResError) as exc:
        B.aggregate_backward(H, w, g, grads, workspace=short)
    assert exc.value.status == B.EINVAL
    coef = torch.zeros((T, Bl, n, 3), dtype=torch.float32, device=dev)
    dws = [torch.zeros(d, dtype=torch.float32, device=dev) for _ in range(Bl)]
    need = B.block_workspace_bytes(T, d, Bl)
    short = torch.empty(max(need // 4 - 4, 4), dtype=torch.float32, device=dev)
    with pytest.raises(B.AttnResError) as exc:
        B.block_backward(H, [g] * Bl, [w] * Bl, coef, grads, dws, workspace=short)
    assert exc.value.status == B.EINVAL
    torch.cuda.synchronize()
    assert not grads.any() and not any(x.any() for x in dws), "nothing may run on a rejected call"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_backward_one_source_passes_the_gradient_through(dtype):
    H, w, g = inputs(1, 50, 264, dtype, seed=8)
    grads = torch.empty((1, 50, 264), dtype=torch.float32, device=H.device)
    dw = B.aggregate_backward(H, w, g, grads)
    torch.cuda.synchronize()
    assert torch.equal(grads[0], g.float())
    assert not dw.any()


def test_backward_empty_batch_zeroes_grad_w():
    dev = device()
    H = torch.empty((3, 0, 256), dtype=torch.bfloat16, device=dev)
    grads = torch.empty((3, 0, 256), dtype=torch.float32, device=dev)
    g = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    gw = torch.full((256,), 7.0, device=dev)
    B.aggregate_backward(H, synth.query(256, device=dev), g, grads, grad_w=gw)
    torch.cuda.synchronize()
    assert not gw.any()


def test_backward_grid_stride_and_strided_rows():
    """More tokens than workgroups, sources and gradients at padded row strides."""
    dev = device()
    S, T, d = 5, 1500, 264
    Hbig, w, g = inputs(S, T + 3, d, torch.bfloat16, seed=10)
    H = Hbig[:, :T]                                      # row stride (T+3)*d
    g = g[:T].contiguous()
    gbig = torch.zeros((S, T + 5, d), dtype=torch.float32, device=dev)
    grads = gbig[:, :T]
    dw = B.aggregate_backward(H, w, g, grads)
    torch.cuda.synchronize()
    check(host(grads), host(dw), host(H), host(w), host(g), "grid-stride")
    assert not gbig[:, T:].any(), "rows past T were written"


def test_backward_last_source_apart_equals_stacked():
    H, w, g = inputs(4, 90, 1024, torch.bfloat16, seed=12)
    dev = H.device
    a = torch.empty((4, 90, 1024), dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    dwa = B.aggregate_backward(H, w, g, a)
    last = H[3].clone()
    dwb = B.aggregate_backward(H[:3], w, g, b, last_source=last)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(dwa, dwb)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_add_rows_is_the_partial_update(dtype):
    dev = device()
    a = synth.layer_output(77, 1032, std=3.0, seed=1, tag=1, device=dev).to(dtype)
    b = synth.layer_output(77, 1032, std=0.01, seed=1, tag=2, device=dev).to(dtype)
    out = torch.empty_like(a)
    B.add_rows(a, b, out)
    copy = torch.empty_like(a)
    B.add_rows(None, b, copy)
    inplace = a.clone()
    B.add_rows(inplace, b, inplace)
    torch.cuda.synchronize()
    ref = orc.accumulate(host(a), host(b), "bf16" if dtype == torch.bfloat16 else "f32")
    assert np.array_equal(host(out), ref) and torch.equal(copy, b) and torch.equal(inplace, out)


def test_backward_full_size_sampled():
    """The bench's backward shape (T = 32768, d = 7168, S = 9): sampled tokens'
    dH against the oracle; dw over a gathered sample against the oracle; and dw
    of the whole batch equal (to float32 rounding) to the sum of dw over two
    halves -- properties that hold at any size."""
    dev = device()
    S, T, d = 9, 32768, 7168
    note("backward full size")
    H, w, g = inputs(S, T, d, torch.bfloat16, seed=21)
    grads = torch.empty((S, T, d), dtype=torch.float32, device=dev)
    dw = B.aggregate_backward(H, w, g, grads)
    rows = synth.token_sample(T, 48, 16, seed=3).to(dev)
    Hs = H.index_select(1, rows).contiguous()
    gs = g.index_select(0, rows).contiguous()
    torch.cuda.synchronize()
    check(host(grads.index_select(1, rows)), None, host(Hs), host(w), host(gs), "full-size sampled dH")
    # dw over exactly the sampled tokens, run on the GPU as a small batch
    small = torch.empty((S, rows.numel(), d), dtype=torch.float32, device=dev)
    dw_small = B.aggregate_backward(Hs, w, gs, small)
    torch.cuda.synchronize()
    check(host(small), host(dw_small), host(Hs), host(w), host(gs), "gathered sample")
    assert torch.equal(small, grads.index_select(1, rows)), "a token's dH depends only on that token"
    # linearity over tokens
    half = T // 2
    g1 = torch.empty((S, half, d), dtype=torch.float32, device=dev)
    dw1 = B.aggregate_backward(H[:, :half], w, g[:half].contiguous(), g1)
    dw2 = B.aggregate_backward(H[:, half:], w, g[half:].contiguous(), g1)
    torch.cuda.synchronize()
    tot = (dw1.double() + dw2.double()).cpu().numpy()
    err = np.max(np.abs(host(dw).astype(np.float64) - tot))
    assert err <= 1e-5 * np.max(np.abs(tot)), f"dw over the batch vs the two halves: {err:.3e}"


def _check_schedule_backward(L, bs, T, d, final, defer, seed):
    """Every gradient of the backward schedule compared with the oracle's
    run_schedule_backward (dF and dh_0 rounded to bf16 when handed out)."""
    dev = device()
    note(f"schedule backward L={L} block={bs} T={T} d={d} final={final} defer={defer}")
    store = B.SourceStore(T, d, dtype=torch.bfloat16, device=dev)
    synth.fill_normal_(store.h0, 1.0, seed=seed, tag=1)
    Fs = [synth.layer_output(T, d, std=0.3, seed=seed, tag=l, device=dev) for l in range(L)]
    Ws = [synth.query(d, seed=seed, device=dev, tag=l) for l in range(L)]
    wf = synth.query(d, seed=seed, device=dev, tag=500)
    gr = [synth.layer_output(T, d, std=1.0, seed=seed, tag=100 + l, device=dev) for l in range(L)]
    gf = synth.layer_output(T, d, std=1.0, seed=seed, tag=999, device=dev)
    schedule.run_schedule(store, Fs, Ws, bs, final_query=wf if final else None)
    handed = {}
    gs, gw, gwf = schedule.run_schedule_backward(
        store, Fs, Ws, bs, gr, final_query=wf if final else None, grad_final=gf if final else None,
        on_grad=lambda l, dF: handed.__setitem__(l, dF.clone()), defer=defer)
    torch.cuda.synchronize()
    ref = orc.run_schedule_backward(host(store.h0), [host(F) for F in Fs], [host(w) for w in Ws], bs, "bf16",
                                    [host(x) for x in gr], final_query=host(wf) if final else None,
                                    grad_final=host(gf) if final else None)
    scale = max(np.max(np.abs(x)) for x in ref["dF"] + [ref["dh0"]])
    # float32 accumulation of up to L+1 aggregations' gradients, then one bf16 rounding
    for l in range(0, L + 1):
        want = ref["dh0"] if l == 0 else ref["dF"][l - 1]
        got = host(handed[l])
        err = np.abs(got - want)
        lim = 2.0 ** -8 * np.abs(want) + 1e-4 * scale
        assert np.all(err <= lim), f"dF_{l}: max error {np.max(err):.3e}"
    err = np.max(np.abs(host(gs[0]) - ref["dh0"]))
    assert err <= 1e-4 * scale, f"dh0 row: {err:.3e}"
    for l in range(L):
        wscale = np.max(np.abs(ref["dw"][l])) + 1e-30
        e = np.max(np.abs(host(gw[l]) - ref["dw"][l]))
        assert e <= 1e-3 * wscale, f"dw layer {l + 1}: {e:.3e} of {wscale:.3e}"
    if final:
        e = np.max(np.abs(host(gwf) - ref["dw_final"]))
        assert e <= 1e-3 * np.max(np.abs(ref["dw_final"])), f"dw final: {e:.3e}"


@pytest.mark.parametrize("defer", [True, False], ids=["deferred", "per_layer"])
@pytest.mark.parametrize("final", [True, False])
def test_schedule_backward_matches_oracle(final, defer):
    """10 layers in blocks of 4; the inter-block gradients deferred to one pass
    per block, or updated per layer."""
    _check_schedule_backward(10, 4, 48, 264, final, defer, 2)


def _random_backward_schedules(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        bs = int(rng.integers(1, 13))
        nblocks = int(rng.integers(1, 9))
        L = int(rng.integers((nblocks - 1) * bs + 1, nblocks * bs + 1))
        out.append((L, bs, int(rng.integers(1, 60)), int(8 * rng.integers(1, 80)), bool(rng.random() < 0.6),
                    bool(rng.random() < 0.7), 40 + k))
    return out


@pytest.mark.parametrize("case", _random_backward_schedules(5, 4321),
                         ids=lambda c: f"L{c[0]}-b{c[1]}-T{c[2]}-d{c[3]}-final{int(c[4])}-defer{int(c[5])}")
def test_random_backward_schedules_match_oracle(case):
    """Seeded random layer counts, block sizes, T and d, with and without the
    output layer and deferral."""
    _check_schedule_backward(*case)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("S,defer,T,d,acc", [(9, 0xFF, 37, 7168, 0), (9, 0xFF, 37, 7168, 0x100),
                                             (4, 0b0101, 45, 1032, 0b1010), (3, 0b111, 20, 264, 0),
                                             (2, 0b01, 300, 7176, 0b10), (1, 0b0, 9, 7168, 1)])
def test_deferred_backward_matches_oracle(dtype, S, defer, T, d, acc):
    """Deferred sources: their rows stay untouched and their coefficients,
    recombined as a_s g + c1_s w - c3_s H_s, give the oracle's dH_s; the other
    rows match the oracle (added into the prefill where ``acc`` says so), the
    handed-out copy of the last row is its rounding, and dL/dw is the oracle's
    share of the other sources."""
    note(f"deferred backward dtype={dtype} S={S} defer={defer:#x} T={T} d={d} acc={acc:#x}")
    H, w, g = inputs(S, T, d, dtype, seed=S * 7 + T)
    dev = H.device
    prefill = torch.randn((S, T, d), generator=torch.Generator(device=dev).manual_seed(5), device=dev)
    grads = prefill.clone()
    coef = torch.full((T, 3 * S), float("nan"), dtype=torch.float32, device=dev)
    last_deferred = (defer >> (S - 1)) & 1
    hand = None if last_deferred else torch.empty((T, d), dtype=dtype, device=dev)
    dw = B.aggregate_backward(H, w, g, grads, accumulate=acc, defer=defer, coef=coef, coef_stride=3 * S,
                              grad_last=hand)
    torch.cuda.synchronize()
    Hh, wh, gh = host(H), host(w), host(g)
    dH_ref, _, dw_src = orc.depth_attention_backward(Hh, wh, gh, per_source=True)
    bH, bw = bounds(Hh, wh, gh)
    cf = host(coef).astype(np.float64).reshape(T, S, 3)
    got = host(grads)
    for s in range(S):
        if (defer >> s) & 1:
            assert torch.equal(grads[s], prefill[s]), f"deferred row {s} was written"
            rec = cf[:, s, 0:1] * gh + cf[:, s, 1:2] * wh[None] - cf[:, s, 2:3] * Hh[s]
        else:
            assert np.all(np.isnan(cf[:, s])), f"coefficients written for source {s}, which is not deferred"
            rec = got[s] - (host(prefill[s]) if (acc >> s) & 1 else 0.0)
        err = np.abs(rec - dH_ref[s])
        lim = C_BWD * bH[s] + 2.0 ** -22 * (np.abs(dH_ref[s]) + np.abs(host(prefill[s])))
        assert np.all(err <= lim), f"source {s}: ratio {np.max(err / lim):.3g}"
    if hand is not None:
        assert torch.equal(hand, grads[S - 1].to(dtype)), "handed-out gradient is not the row's rounding"
    share = sum(dw_src[s] for s in range(S) if not (defer >> s) & 1) if defer != (1 << S) - 1 else np.zeros(d)
    errw = np.abs(host(dw).astype(np.float64) - share)
    limw = C_BWD * bw + 2.0 ** -23 * np.abs(share)
    assert np.all(errw <= limw), f"dw share: ratio {np.max(errw / limw):.3g}"


def test_block_backward_equals_per_layer_updates():
    """One block of B = 6 layers over n = 5 inter-block sources (+ a partial):
    deferring the inter-block gradients to attnres_block_backward gives the
    per-layer result up to float32 summation order -- the gradient rows and,
    once the block pass adds the deferred sources' share, dL/dw; the partial's
    gradient row is identical."""
    dev = device()
    n, Bl, T, d = 5, 6, 70, 1032
    H, _, _ = inputs(n, T, d, torch.bfloat16, seed=31)
    part = synth.layer_output(T, d, std=2.0, seed=31, tag=9, device=dev)
    Ws = [synth.query(d, seed=31, device=dev, tag=l) for l in range(Bl)]
    Gs = [synth.layer_output(T, d, std=1.0, seed=31, tag=50 + l, device=dev) for l in range(Bl)]
    prefill = torch.randn((n + 1, T, d), generator=torch.Generator(device=dev).manual_seed(4), device=dev)
    ref = prefill.clone()
    got = prefill.clone()
    coef = torch.empty((T, Bl, n, 3), dtype=torch.float32, device=dev)
    dws_ref, dws_got = [], []
    last_ref = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    last_got = torch.empty_like(last_ref)
    for l in range(Bl):
        dws_ref.append(B.aggregate_backward(H, Ws[l], Gs[l], ref, last_source=part, accumulate=(1 << (n + 1)) - 1,
                                            grad_last=last_ref))
        dws_got.append(B.aggregate_backward(H, Ws[l], Gs[l], got, last_source=part, accumulate=(1 << (n + 1)) - 1,
                                            defer=(1 << n) - 1, coef=coef.view(-1)[3 * n * l:],
                                            coef_stride=3 * n * Bl, grad_last=last_got))
    torch.cuda.synchronize()
    assert torch.equal(last_ref, last_got) and torch.equal(ref[n], got[n]), "partial row"
    assert torch.equal(got[:n], prefill[:n]), "deferred rows must be untouched before the block pass"
    emit = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    B.block_backward(H, Gs, Ws, coef, got[:n], dws_got, accumulate=(1 << n) - 1, grad_last=emit)
    torch.cuda.synchronize()
    diff = (got[:n] - ref[:n]).abs().max().item()
    scale = ref[:n].abs().max().item()
    assert diff <= 1e-5 * scale, f"deferred vs per-layer: {diff:.3e} of {scale:.3e}"
    assert torch.equal(emit, got[n - 1].to(torch.bfloat16))
    for l in range(Bl):
        e = (dws_got[l] - dws_ref[l]).abs().max().item()
        assert e <= 1e-4 * dws_ref[l].abs().max().item(), f"dL/dw layer {l}: {e:.3e}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("n,Bl,T,d", [(1, 1, 9, 8), (8, 16, 33, 2056), (3, 13, 300, 7168), (7, 2, 5, 1024)])
def test_block_backward_matches_oracle(dtype, n, Bl, T, d):
    """attnres_block_backward on coefficients the oracle fixes: for each layer
    the per-layer coefficients are those of an aggregation over the n sources
    (written by a deferred attnres_aggregate_backward, checked above), and the
    block pass must leave each G_s equal to prefill + sum_l dH_{l,s} of the
    oracle and add each layer's full dL/dw -- shapes with a ragged d slice, the
    most layers and sources, and a single element group."""
    note(f"block backward dtype={dtype} n={n} B={Bl} T={T} d={d}")
    H, _, _ = inputs(n, T, d, dtype, seed=n * 31 + Bl)
    dev = H.device
    name = "bf16" if dtype == torch.bfloat16 else "f32"
    Ws = [synth.query(d, seed=n, device=dev, tag=l) for l in range(Bl)]
    Gs = [synth.layer_output(T, d, std=1.0, seed=n, tag=60 + l, device=dev, dtype=name) for l in range(Bl)]
    prefill = torch.randn((n, T, d), generator=torch.Generator(device=dev).manual_seed(6), device=dev)
    grads = prefill.clone()
    coef = torch.empty((T, Bl, n, 3), dtype=torch.float32, device=dev)
    scratch = torch.zeros((n, T, d), dtype=torch.float32, device=dev)
    dws = []
    for l in range(Bl):
        dws.append(B.aggregate_backward(H, Ws[l], Gs[l], scratch, defer=(1 << n) - 1,
                                        coef=coef.view(-1)[3 * n * l:], coef_stride=3 * n * Bl))
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


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("S,defer,T,d,acc", [(9, 0xFF, 37, 7168, 0x100), (9, 0, 37, 7168, 0x1FF),
                                             (4, 0b0101, 45, 1032, 0b1010), (3, 0b111, 20, 264, 0),
                                             (2, 0b01, 300, 7176, 0b10), (1, 0b0, 9, 7168, 1)])
def test_backward_without_dw_matches_oracle_and_the_dw_form(dtype, S, defer, T, d, acc):
    """grad_w NULL (dL/dw left to the caller, one workgroup per token): the
    gradient rows, the handed-out copy and the deferred sources' coefficients
    are those of the dL/dw form bit for bit; every source's coefficients are
    written, the non-deferred ones recombine to the oracle's dH_s, and their
    c1 summed over tokens with the rows (float64, on the host) is the oracle's
    dL/dw share of those sources."""
    note(f"backward without dw dtype={dtype} S={S} defer={defer:#x} T={T} d={d} acc={acc:#x}")
    H, w, g = inputs(S, T, d, dtype, seed=S * 5 + T)
    dev = H.device
    prefill = torch.randn((S, T, d), generator=torch.Generator(device=dev).manual_seed(8), device=dev)
    last_deferred = (defer >> (S - 1)) & 1
    runs = []
    for form_dw in (True, False):
        grads = prefill.clone()
        coef = torch.full((T, 3 * S), float("nan"), dtype=torch.float32, device=dev)
        hand = None if last_deferred else torch.empty((T, d), dtype=dtype, device=dev)
        kw = dict(coef=coef, coef_stride=3 * S) if (defer or not form_dw) else {}
        dw = B.aggregate_backward(H, w, g, grads, accumulate=acc, defer=defer, grad_last=hand, form_dw=form_dw, **kw)
        runs.append((grads, coef, hand, dw))
    torch.cuda.synchronize()
    (ga, ca, ha, dwa), (gb, cb, hb, dwb) = runs
    assert dwb is None
    assert torch.equal(ga, gb), "gradient rows differ between the two forms"
    if ha is not None:
        assert torch.equal(ha, hb), "handed-out gradient differs"
    cfa = host(ca).reshape(T, S, 3)
    cf = host(cb).astype(np.float64).reshape(T, S, 3)
    assert not np.any(np.isnan(cf)), "a source's coefficients were not written"
    Hh, wh, gh = host(H), host(w), host(g)
    dH_ref, _, dw_src = orc.depth_attention_backward(Hh, wh, gh, per_source=True)
    bH, bw = bounds(Hh, wh, gh)
    share = np.zeros(d)
    for s in range(S):
        if (defer >> s) & 1:
            assert np.array_equal(cfa[:, s].view(np.int32), host(cb).reshape(T, S, 3)[:, s].view(np.int32)), \
                f"coefficients of deferred source {s} differ"
            continue
        rec = cf[:, s, 0:1] * gh + cf[:, s, 1:2] * wh[None] - cf[:, s, 2:3] * Hh[s]
        err = np.abs(rec - dH_ref[s])
        lim = C_BWD * bH[s] + 2.0 ** -22 * np.abs(dH_ref[s])
        assert np.all(err <= lim), f"coefficients of source {s}: ratio {np.max(err / lim):.3g}"
        share += dw_src[s]
    mine = sum(cf[:, s, 1] @ Hh[s] for s in range(S) if not (defer >> s) & 1) if defer != (1 << S) - 1 else 0.0
    errw = np.abs(mine - share)
    limw = C_BWD * bw + 2.0 ** -23 * np.abs(share) + np.finfo(np.float32).tiny
    assert np.all(errw <= limw), f"dw share from the coefficients: ratio {np.max(errw / limw):.3g}"


def test_backward_without_dw_empty_batch_launches_nothing():
    dev = device()
    H = torch.empty((3, 0, 264), dtype=torch.bfloat16, device=dev)
    grads = torch.empty((3, 0, 264), dtype=torch.float32, device=dev)
    coef = torch.empty(9, dtype=torch.float32, device=dev)
    B.aggregate_backward(H, synth.query(264, device=dev), torch.empty((0, 264), dtype=torch.bfloat16, device=dev),
                         grads, defer=0b011, coef=coef, coef_stride=9, form_dw=False)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("T,d,Bl", [(1, 8, 1), (37, 264, 3), (1000, 7168, 12), (4099, 520, 16), (32768, 7168, 2)])
def test_partial_dw_matches_float64(dtype, T, d, Bl):
    """attnres_partial_dw: grad_ws[l] = sum_t c_l[t] X_l[t] for the layers with a
    row (layer 0 and every third have none and get zeros), coefficients read
    at an odd layer stride from mid-buffer, against a float64 sum on the host
    (all columns, or 256 sampled ones at T = 32,768); bitwise equal on a
    second call.  The float32 sum runs over token groups and then the groups:
    its error is far below 1e-4 of sum |c x|."""
    dev = device()
    note(f"partial dw dtype={dtype} T={T} d={d} B={Bl}")
    name = "bf16" if dtype == torch.bfloat16 else "f32"
    rows = [None if (l % 3 == 0) else synth.layer_output(T, d, std=1.5, seed=T + l, tag=300 + l, device=dev,
                                                          dtype=name) for l in range(Bl)]
    m = 7
    gen = torch.Generator(device=dev).manual_seed(T + Bl)
    coef = torch.randn((T * Bl * m + 8,), generator=gen, device=dev) * torch.exp(
        torch.randn((T * Bl * m + 8,), generator=gen, device=dev))
    base = coef[4:]
    outs = []
    for _ in range(2):
        dws = [torch.full((d,), float("nan"), dtype=torch.float32, device=dev) for _ in range(Bl)]
        B.partial_dw(rows, base, Bl * m, m, dws)
        outs.append(dws)
    torch.cuda.synchronize()
    cols = np.arange(d) if T * d <= 8 << 20 else np.sort(np.random.default_rng(T).choice(d, 256, replace=False))
    c = host(base)[: T * Bl * m].astype(np.float64).reshape(T, Bl, m)[:, :, 0]
    for l in range(Bl):
        assert torch.equal(outs[0][l], outs[1][l]), f"layer {l}: not reproducible"
        got = host(outs[0][l]).astype(np.float64)
        if rows[l] is None:
            assert np.all(got == 0.0), f"layer {l} has no row: its dL/dw share must be zero"
            continue
        X = host(rows[l][:, torch.as_tensor(cols, device=dev)]).astype(np.float64)
        want = c[:, l] @ X
        mag = np.abs(c[:, l]) @ np.abs(X)
        err = np.abs(got[cols] - want)
        assert np.all(err <= 1e-4 * mag + 1e-30), f"layer {l}: ratio {np.max(err / (1e-4 * mag + 1e-30)):.3g}"


def test_partial_dw_empty_batch_zeroes_the_rows():
    dev = device()
    dws = [torch.full((264,), 3.0, dtype=torch.float32, device=dev) for _ in range(3)]
    rows = [None, torch.empty((0, 264), dtype=torch.bfloat16, device=dev), None]
    B.partial_dw(rows, None, 9, 3, dws)
    torch.cuda.synchronize()
    assert all(torch.equal(x, torch.zeros_like(x)) for x in dws)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("n,Bl,T,d", [(1, 3, 9, 8), (5, 12, 77, 1032), (8, 16, 33, 2056)])
def test_block_backward_layer_stride_is_the_packed_layout(dtype, n, Bl, T, d):
    """attnres_block_backward with m = 3(n + 1) floats per layer slot (a layer's
    own last source's triple after the n inter-block ones, filled with
    garbage here) gives the packed [T][B][n][3] layout's results bit for bit:
    gradient rows, handed-out row and every layer's dL/dw."""
    dev = device()
    note(f"block backward layer stride dtype={dtype} n={n} B={Bl} T={T} d={d}")
    H, _, _ = inputs(n, T, d, dtype, seed=n + Bl)
    name = "bf16" if dtype == torch.bfloat16 else "f32"
    Ws = [synth.query(d, seed=n, device=dev, tag=l) for l in range(Bl)]
    Gs = [synth.layer_output(T, d, std=1.0, seed=n, tag=70 + l, device=dev, dtype=name) for l in range(Bl)]
    gen = torch.Generator(device=dev).manual_seed(n * Bl)
    wide = torch.randn((T, Bl, n + 1, 3), generator=gen, device=dev) * 1e-2
    packed = wide[:, :, :n].contiguous()
    wide[:, :, n] = 1e30                               # never read
    prefill = torch.randn((n, T, d), generator=gen, device=dev)
    res = []
    for coef, m in ((packed, 0), (wide, 3 * (n + 1))):
        grads = prefill.clone()
        dws = [torch.full((d,), 0.25, dtype=torch.float32, device=dev) for _ in range(Bl)]
        emit = torch.empty((T, d), dtype=dtype, device=dev)
        B.block_backward(H, Gs, Ws, coef, grads, dws, accumulate=(1 << n) - 1, grad_last=emit, coef_layer_stride=m)
        res.append((grads, dws, emit))
    torch.cuda.synchronize()
    (g0, w0, e0), (g1, w1, e1) = res
    assert torch.equal(g0, g1) and torch.equal(e0, e1)
    assert all(torch.equal(a, b) for a, b in zip(w0, w1))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("count", [1, 2, 11, 16])
def test_partial_sums_are_the_store_updates(dtype, count):
    """attnres_partial_sums equals the oracle's update chain bit for bit."""
    dev = device()
    T, d = 37, 520
    name = "bf16" if dtype == torch.bfloat16 else "f32"
    Fs = [synth.layer_output(T, d, std=0.1 + k, seed=4, tag=k, device=dev, dtype=name) for k in range(count)]
    out = torch.empty((16, T, d), dtype=dtype, device=dev)
    B.partial_sums(Fs, out)
    torch.cuda.synchronize()
    part = None
    for k in range(count):
        part = orc.accumulate(part, host(Fs[k]), name)
        assert np.array_equal(host(out[k]), part), f"partial {k}"


@pytest.mark.parametrize("case", ["zero_query", "identical_sources", "tiny_source", "zero_source", "huge_query"])
def test_backward_degenerate_cases(case):
    """The method's degenerate inputs through the backward, against the oracle
    within the same bound: a zero query (uniform weights, no key-path term from
    the logits), identical sources (equal logits), a source whose mean square
    is near eps, an all-zero source (key 0, logit 0), and a huge query
    (one-hot weights, the softmax gradient vanishing)."""
    note(f"backward degenerate {case}")
    S, T, d = 5, 40, 1032
    H, w, g = inputs(S, T, d, torch.float32, seed=44)
    if case == "zero_query":
        w = torch.zeros_like(w)
    elif case == "identical_sources":
        H = H[:1].repeat(S, 1, 1).contiguous()
    elif case == "tiny_source":
        H[2] *= 3e-3 / H[2].pow(2).mean(dim=-1, keepdim=True).sqrt()
    elif case == "zero_source":
        H[1].zero_()
    elif case == "huge_query":
        w = w * 1e4
    grads = torch.empty((S, T, d), dtype=torch.float32, device=H.device)
    dw = B.aggregate_backward(H, w, g, grads)
    torch.cuda.synchronize()
    check(host(grads), host(dw), host(H), host(w), host(g), f"degenerate {case}")
    assert torch.isfinite(grads).all() and torch.isfinite(dw).all()
