"""The oracle's backward against what the mathematics fixes (CPU only).

Each backward pin must pass; each planted mistake (a copy of the oracle's
backward arithmetic with one plausible error) must fail at least one pin; and
the schedule backward must equal torch autograd through the whole Block
AttnRes schedule built from library routines.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attnres_oracle as orc
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.BACKWARD_PINS, ids=lambda p: p.__name__)
def test_oracle_backward_passes_pin(pin):
    pin(orc.depth_attention_backward)


def _mutant(key_sign=-1.0, centre=True, weight_factor=True, dw_from="keys", project=True, value="a_g"):
    def bwd(H, w, g, eps):
        H = np.asarray(H, np.float64)
        w = np.asarray(w, np.float64)
        g = np.asarray(g, np.float64)
        S, T, d = H.shape
        rms = np.sqrt(np.mean(H * H, -1, keepdims=True) + eps)
        keys = H / rms
        a = orc.softmax((keys @ w).T, axis=1)
        da = np.stack([np.sum(g * H[s], axis=1) for s in range(S)], axis=1)
        centred = da - np.sum(a * da, axis=1, keepdims=True) if centre else da
        dz = a * centred if weight_factor else centred
        src = keys if dw_from == "keys" else H
        dw = sum(np.sum(dz[:, s:s + 1] * src[s], axis=0) for s in range(S))
        dkeys = np.stack([dz[:, s:s + 1] * w for s in range(S)])
        proj = np.mean(dkeys * keys, -1, keepdims=True) if project else 0.0
        dH = (dkeys + key_sign * keys * proj) / rms
        for s in range(S):
            if value == "a_g":
                dH[s] += a[:, s:s + 1] * g
            elif value == "a_g_over_rms":
                dH[s] += a[:, s:s + 1] * g / rms[s]
        return dH, dw
    return bwd


MUTANTS = {
    "key_projection_sign": _mutant(key_sign=+1.0),
    "softmax_not_centred": _mutant(centre=False),
    "softmax_without_weight": _mutant(weight_factor=False),
    "query_gradient_from_raw_sources": _mutant(dw_from="raw"),
    "rmsnorm_without_projection": _mutant(project=False),
    "value_path_normalised": _mutant(value="a_g_over_rms"),
    "value_path_missing": _mutant(value="none"),
}


def test_mutant_builder_reproduces_the_oracle():
    """The unmodified copy equals the oracle, so each mutant differs by one mistake."""
    rng = np.random.default_rng(0)
    H = rng.normal(size=(4, 3, 16))
    w = rng.normal(size=16)
    g = rng.normal(size=(3, 16))
    dH, dw = _mutant()(H, w, g, orc.EPS)
    dH0, dw0 = orc.depth_attention_backward(H, w, g)
    assert np.allclose(dH, dH0, rtol=1e-13, atol=0) and np.allclose(dw, dw0, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_backward_mistake_is_caught(name):
    failures = []
    for pin in pins.BACKWARD_PINS:
        try:
            pin(MUTANTS[name])
        except AssertionError as exc:
            failures.append(f"{pin.__name__}: {exc}")
    assert failures, f"planted mistake {name!r} passed every backward pin"


def test_oracle_per_source_query_shares_pinned():
    def shares(H, w, g, eps):
        _, dw, dw_src = orc.depth_attention_backward(H, w, g, eps, per_source=True)
        return dw, dw_src
    pins.pin_backward_per_source(shares)


def test_planted_per_source_mistake_is_caught():
    """Shares taken along the raw sources instead of the keys fail the pin."""
    def wrong(H, w, g, eps):
        H = np.asarray(H, np.float64)
        _, dw = orc.depth_attention_backward(H, w, g, eps)
        _, a = orc.depth_attention(H, w, eps)
        da = np.stack([np.sum(np.asarray(g) * H[s], axis=1) for s in range(H.shape[0])], axis=1)
        dz = a * (da - np.sum(a * da, axis=1, keepdims=True))
        raw = np.stack([np.sum(dz[:, s:s + 1] * H[s], axis=0) for s in range(H.shape[0])])
        return dw, raw
    with pytest.raises(AssertionError):
        pins.pin_backward_per_source(wrong)


def _torch_schedule_grads(h0, Fs, Ws, block_size, g_r, w_final, g_final, eps=orc.EPS):
    """Autograd through Block AttnRes written with torch sums, rms_norm and sdpa
    in float64 (exact sums: the inputs are small integers)."""
    h0t = torch.tensor(h0, dtype=torch.float64, requires_grad=True)
    Ft = [torch.tensor(F_, dtype=torch.float64, requires_grad=True) for F_ in Fs]
    Wt = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in Ws]
    wf = torch.tensor(w_final, dtype=torch.float64, requires_grad=True)
    T, d = h0.shape

    def agg(srcs, w):
        H = torch.stack(srcs)                                   # [S, T, d]
        keys = F.rms_norm(H, (d,), eps=eps).permute(1, 0, 2)
        q = w.view(1, 1, d).expand(T, 1, d)
        return F.scaled_dot_product_attention(q, keys, H.permute(1, 0, 2), scale=1.0)[:, 0, :]

    L = len(Fs)
    loss = 0.0
    blocks = []
    for l in range(1, L + 1):
        n, i = (l - 1) // block_size + 1, (l - 1) % block_size + 1
        first = (n - 1) * block_size
        srcs = [h0t] + blocks
        if i >= 2:
            srcs = srcs + [sum(Ft[first:l - 1])]
        loss = loss + (agg(srcs, Wt[l - 1]) * torch.tensor(g_r[l - 1])).sum()
        if i == block_size or l == L:
            blocks.append(sum(Ft[first:l]))
    loss = loss + (agg([h0t] + blocks, wf) * torch.tensor(g_final)).sum()
    loss.backward()
    return h0t.grad.numpy(), [f.grad.numpy() for f in Ft], [w.grad.numpy() for w in Wt], wf.grad.numpy()


@pytest.mark.parametrize("L,block_size", [(7, 3), (5, 1), (6, 6)])
def test_schedule_backward_equals_autograd(L, block_size):
    rng = np.random.default_rng(L * 10 + block_size)
    T, d = 3, 16
    h0 = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    Fs = [rng.integers(-4, 5, size=(T, d)).astype(np.float32) for _ in range(L)]
    Ws = [rng.normal(scale=0.5, size=d) for _ in range(L)]
    wf = rng.normal(scale=0.5, size=d)
    g_r = [rng.normal(size=(T, d)) for _ in range(L)]
    g_f = rng.normal(size=(T, d))
    got = orc.run_schedule_backward(h0, Fs, Ws, block_size, "bf16", g_r, final_query=wf, grad_final=g_f)
    dh0, dF, dW, dwf = _torch_schedule_grads(h0, Fs, Ws, block_size, g_r, wf, g_f)
    np.testing.assert_allclose(got["dh0"], dh0, rtol=1e-11, atol=1e-12)
    for l in range(L):
        np.testing.assert_allclose(got["dF"][l], dF[l], rtol=1e-11, atol=1e-12, err_msg=f"dF layer {l + 1}")
        np.testing.assert_allclose(got["dw"][l], dW[l], rtol=1e-11, atol=1e-12, err_msg=f"dw layer {l + 1}")
    np.testing.assert_allclose(got["dw_final"], dwf, rtol=1e-11, atol=1e-12)


def test_schedule_backward_hand_out_is_by_membership():
    """Structural: with every upstream gradient zero but one layer's, only that
    layer's sources receive gradient -- h_0, the earlier blocks' layers and the
    same block's earlier layers, nothing after it."""
    rng = np.random.default_rng(5)
    T, d, L, bs = 2, 8, 8, 3
    h0 = rng.normal(size=(T, d)).astype(np.float32)
    Fs = [rng.normal(size=(T, d)).astype(np.float32) for _ in range(L)]
    Ws = [rng.normal(size=d) for _ in range(L)]
    layer = 6                                    # block 2, position 3
    g_r = [np.zeros((T, d)) if l + 1 != layer else rng.normal(size=(T, d)) for l in range(L)]
    got = orc.run_schedule_backward(h0, Fs, Ws, bs, "f32", g_r)
    touched = [bool(np.any(x != 0)) for x in got["dF"]]
    assert touched == [True, True, True, True, True, False, False, False]
    assert np.any(got["dh0"] != 0)
