"""bf16 rounding, the partial-sum update and the block schedule of the oracle,
pinned against torch, hand-derived rounding cases and the pages' source counts."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attnres_oracle as orc
from tests.oracle_pins import GOLDEN


def _hex(s):
    return int(s, 16)


def test_bf16_rounding_hand_cases():
    with open(os.path.join(GOLDEN, "bf16_rne_cases.json")) as f:
        cases = json.load(f)["cases"]
    bits = np.array([_hex(c["f32"]) for c in cases], np.uint32)
    got = orc.f32_to_bf16_bits(bits.view(np.float32))
    for c, g in zip(cases, got):
        if c["bf16"] == "nan":
            assert (g & 0x7F80) == 0x7F80 and (g & 0x007F) != 0, c["why"]
        else:
            assert int(g) == _hex(c["bf16"]), f'{c["f32"]}: {c["why"]} (got {int(g):#06x})'


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(size=200_000).astype(np.float32) * np.float32(10) ** rng.integers(-30, 30, 200_000).astype(np.float32),
        rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[~np.isnan(x)]
    ours = orc.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(orc.bf16_round(x).view(np.uint32) & 0xFFFF, np.zeros(x.size, np.uint32))


def test_accumulate_bf16_matches_torch_float32_add_then_round():
    rng = np.random.default_rng(1)
    n = 300_000
    p = orc.bf16_round((rng.normal(size=n) * np.exp(rng.uniform(-8, 8, n))).astype(np.float32))
    F = orc.bf16_round((rng.normal(size=n) * np.exp(rng.uniform(-8, 8, n))).astype(np.float32))
    got = orc.accumulate(p, F, "bf16")
    ref = (torch.from_numpy(p) + torch.from_numpy(F)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_accumulate_first_layer_is_a_copy_and_f32_is_a_plain_add():
    rng = np.random.default_rng(2)
    F = orc.bf16_round(rng.normal(size=1000).astype(np.float32))
    c = orc.accumulate(None, F, "bf16")
    assert np.array_equal(c.view(np.uint32), F.view(np.uint32)) and c is not F
    p = rng.normal(size=1000).astype(np.float32)
    G = rng.normal(size=1000).astype(np.float32)
    got = orc.accumulate(p, G, "f32")
    assert got.dtype == np.float32
    assert np.array_equal(got, (torch.from_numpy(p) + torch.from_numpy(G)).numpy())
    with pytest.raises(ValueError):
        orc.accumulate(p, G, "fp16")


def _k3():
    with open(os.path.join(GOLDEN, "k3_block_schedule.json")) as f:
        return json.load(f)


def test_k3_layout_matches_the_pages():
    g = _k3()
    layout = orc.block_layout(g["layers"], g["block_size"])
    blocks = sorted({n for n, _ in layout})
    assert len(blocks) == g["blocks"] == math.ceil(g["layers"] / g["block_size"])
    sizes = [sum(1 for n, _ in layout if n == b) for b in blocks]
    assert sizes[:-1] == [g["block_size"]] * (g["blocks"] - 1) and sizes[-1] < g["block_size"]
    counts = [len(orc.layer_source_names(n, i)) for n, i in layout]
    assert counts[0] == g["first_layer_sources"]
    assert max(counts) == g["max_sources_with_embedding"]
    # the output layer sees h0 and every block representation
    assert 1 + g["blocks"] == g["max_sources_with_embedding"]
    # histogram implied by the rule: block n's first layer has n sources, its
    # other layers n + 1
    hist = {s: counts.count(s) for s in sorted(set(counts))}
    assert hist == {1: 1, 2: 12, 3: 12, 4: 12, 5: 12, 6: 12, 7: 12, 8: 12, 9: 8}


def test_layer_sources_have_no_zero_partial():
    assert orc.layer_source_names(1, 1) == ["h0"]
    assert orc.layer_source_names(3, 1) == ["h0", "b1", "b2"]
    assert orc.layer_source_names(3, 2) == ["h0", "b1", "b2", "partial"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_schedule_with_integer_outputs_is_exact(dtype):
    """Small-integer layer outputs make every partial and block sum exact, so the
    schedule can be checked against integer arithmetic."""
    rng = np.random.default_rng(3)
    L, B, T, d = 29, 6, 3, 8
    h0 = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    Fs = rng.integers(-3, 4, size=(L, T, d)).astype(np.float32)
    Ws = rng.normal(scale=0.7, size=(L, d))
    w_out = rng.normal(scale=0.7, size=d)
    out = orc.run_schedule(h0, Fs, Ws, B, dtype, final_query=w_out)
    assert np.array_equal(out["r"][0], h0.astype(np.float64))
    assert out["num_sources"][0] == 1
    blocks = [Fs[k:k + B].sum(axis=0) for k in range(0, L, B)]
    assert len(out["blocks"]) == len(blocks) == math.ceil(L / B)
    for got, ref in zip(out["blocks"], blocks):
        assert np.array_equal(got, ref)
    # layer l at position i >= 2 sees partial = sum of the block's earlier outputs
    for l, (n, i) in enumerate(orc.block_layout(L, B), start=1):
        H = [h0] + blocks[:n - 1]
        if i >= 2:
            start = (n - 1) * B
            H.append(Fs[start:l - 1].sum(axis=0))
        r, a = orc.depth_attention(np.stack(H), Ws[l - 1])
        assert out["num_sources"][l - 1] == len(H)
        assert np.array_equal(out["r"][l - 1], r) and np.array_equal(out["a"][l - 1], a)
    r, a = orc.depth_attention(np.stack([h0] + blocks), w_out)
    assert np.array_equal(out["final_r"], r)


def test_full_attnres_is_block_attnres_with_one_layer_per_block():
    """kimi.papertok.ai ch. 4 §4.3: the L layers are cut into N blocks of L/N
    layers; with N = L every block is one layer, its representation is that
    layer's output, and Block AttnRes reduces to Full AttnRes (§4.2)."""
    rng = np.random.default_rng(5)
    L, T, d = 11, 4, 16
    h0 = orc.bf16_round(rng.normal(size=(T, d)).astype(np.float32))
    Fs = orc.bf16_round(rng.normal(size=(L, T, d)).astype(np.float32))
    Ws = rng.normal(scale=0.5, size=(L, d))
    w_out = rng.normal(scale=0.5, size=d)
    full, final = orc.run_full_schedule(h0, Fs, Ws, final_query=w_out)
    block = orc.run_schedule(h0, Fs, Ws, 1, "bf16", final_query=w_out)
    assert [a.shape[1] for _, a in full] == list(range(1, L + 1)) == block["num_sources"]
    for l in range(L):
        assert np.array_equal(full[l][0], block["r"][l]) and np.array_equal(full[l][1], block["a"][l])
    assert np.array_equal(final[0], block["final_r"]) and final[1].shape == (T, L + 1)


def test_many_sources_match_the_library_reduction():
    """94 sources (Full AttnRes at K3's depth) against torch's RMSNorm + SDPA."""
    from tests.oracle_pins import library_reference
    rng = np.random.default_rng(6)
    H = rng.normal(size=(94, 5, 32)) * rng.uniform(0.1, 10, size=(94, 1, 1))
    w = rng.normal(scale=0.3, size=32)
    r, a = orc.depth_attention(H, w)
    r_lib, a_lib = library_reference(H, w)
    assert np.max(np.abs(a - a_lib)) < 1e-12
    assert np.max(np.abs(r - r_lib)) < 1e-12 * np.max(np.abs(r_lib))
