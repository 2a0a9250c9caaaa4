"""Non-finite inputs stay inside their token.  The pages do not say what a NaN or
an infinity in a source should produce; the kernels leave it to the token's own
arithmetic.  What must hold is independence: a NaN or infinity in one token's
rows changes nothing in any other token -- no shared LDS, workgroup loop or
fused update may carry it across.  Each case compares a run with the planted
value against a clean run, bit for bit, on every other token."""

import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import synth
from tests.gpu_util import device, note

pytestmark = pytest.mark.gpu

VALUES = {"nan": float("nan"), "inf": float("inf"), "-inf": float("-inf")}


def _others(x: torch.Tensor, t: int, dim: int) -> torch.Tensor:
    """x without index t along dim (a copy)."""
    keep = [i for i in range(x.shape[dim]) if i != t]
    return x.index_select(dim, torch.tensor(keep, device=x.device))


@pytest.mark.parametrize("value", list(VALUES))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S", [2, 4, 9, 12])
def test_aggregate_keeps_non_finite_in_its_token(value, dtype, S):
    T, d, bad_t = 600, 1032, 311
    note(f"non-finite aggregate {value} {dtype} S={S}")
    dev = device()
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=S, dtype=dtype, device=dev)
    w = synth.query(d, seed=S, device=dev)
    clean_out, clean_a = B.aggregate(H, w)
    Hb = H.clone()
    Hb[S // 2, bad_t, d // 3] = VALUES[value]
    out, a = B.aggregate(Hb, w)
    torch.cuda.synchronize()
    assert torch.equal(_others(out, bad_t, 0), _others(clean_out, bad_t, 0)), "another token's residual changed"
    assert torch.equal(_others(a, bad_t, 0), _others(clean_a, bad_t, 0)), "another token's weights changed"
    assert not torch.isfinite(a[bad_t]).all() or not torch.isfinite(out[bad_t].float()).all(), \
        "the planted value left no trace in its own token"


@pytest.mark.parametrize("value", list(VALUES))
def test_fused_update_keeps_non_finite_in_its_token(value):
    """A non-finite layer output: the store's partial row and the fused
    aggregation change only at that token."""
    T, d, bad_t = 500, 7168, 123
    note(f"non-finite fused update {value}")
    dev = device()
    stores = [B.SourceStore(T, d, s_max=9, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    init = synth.sources(9, T, d, scale=(0.5, 50.0), seed=7, device=dev)
    for st in stores:
        st.slots.copy_(init)
        st.set_state(4, True)
    F = synth.layer_output(T, d, std=1.0, seed=7, tag=3, device=dev)
    Fb = F.clone()
    Fb[bad_t, 17] = VALUES[value]
    w = synth.query(d, seed=7, device=dev)
    clean_out, clean_a = stores[0].accumulate_aggregate(F, False, w)
    out, a = stores[1].accumulate_aggregate(Fb, False, w)
    torch.cuda.synchronize()
    assert torch.equal(_others(stores[0].slots, bad_t, 1), _others(stores[1].slots, bad_t, 1))
    assert torch.equal(_others(out, bad_t, 0), _others(clean_out, bad_t, 0))
    assert torch.equal(_others(a, bad_t, 0), _others(clean_a, bad_t, 0))


@pytest.mark.parametrize("value", list(VALUES))
@pytest.mark.parametrize("defer", [0, 0b0111], ids=["general", "last_source"])
def test_backward_keeps_non_finite_in_its_token_rows(value, defer):
    """The backward's per-token results (gradient rows, coefficients, the
    handed-out copy) change only at the token with the planted value; dL/dw,
    a sum over tokens, is not checked."""
    S, T, d, bad_t = 4, 700, 1032, 444
    note(f"non-finite backward {value} defer={defer:#x}")
    dev = device()
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=11, device=dev)
    w = synth.query(d, seed=11, device=dev)
    g = synth.layer_output(T, d, std=1.0, seed=11, tag=4, device=dev)
    Hb = H.clone()
    Hb[1, bad_t, 5] = VALUES[value]
    runs = []
    for src in (H, Hb):
        grads = torch.zeros((S, T, d), dtype=torch.float32, device=dev)
        coef = torch.zeros((T, 3 * S), dtype=torch.float32, device=dev)
        hand = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
        B.aggregate_backward(src, w, g, grads, defer=defer, coef=coef if defer else None, coef_stride=3 * S,
                             grad_last=hand)
        runs.append((grads, coef, hand))
    torch.cuda.synchronize()
    (g0, c0, h0), (g1, c1, h1) = runs
    assert torch.equal(_others(g0, bad_t, 1), _others(g1, bad_t, 1)), "another token's gradient rows changed"
    assert torch.equal(_others(c0, bad_t, 0), _others(c1, bad_t, 0)), "another token's coefficients changed"
    assert torch.equal(_others(h0, bad_t, 0), _others(h1, bad_t, 0)), "another token's handed-out gradient changed"
