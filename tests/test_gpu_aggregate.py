"""GPU parity of attnres_aggregate against the oracle: ragged shapes, every
source count, both dtypes, the worked example and the degenerate cases."""

import math

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import synth
from tests import oracle_pins
from tests.gpu_util import compare, device, host, note, oracle_aggregate, same_bits

pytestmark = pytest.mark.gpu


def run(H: torch.Tensor, w: torch.Tensor, **kw):
    out, a = B.aggregate(H, w, **kw)
    torch.cuda.synchronize()
    return out, a


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,T,d", [
    (1, 5, 256), (2, 3, 8), (3, 17, 264), (4, 64, 256), (5, 33, 1000), (6, 7, 7176),
    (7, 129, 2048), (8, 2, 7168), (9, 37, 7168), (9, 11, 4104), (9, 5, 10000), (2, 3, 16384),
])
def test_ragged_shapes_match_oracle(dtype, S, T, d):
    dev = device()
    note(f"aggregate {dtype} S={S} T={T} d={d}")
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=S * 131 + T, dtype=dtype, device=dev)
    w = synth.query(d, seed=T, device=dev)
    if dtype == "f32" and d > B.MAX_D_F32:
        # float32 rows wider than the supported maximum are refused before any launch
        with pytest.raises(B.AttnResError) as exc:
            run(H, w)
        assert exc.value.status == B.EUNSUPPORTED
        return
    out, a = run(H, w)
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(host(out), host(a), r_ref, a_ref, dtype == "bf16", f"{dtype} S={S} T={T} d={d}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_example_weights(dtype):
    """The four-source walk-through of "Kimi K3技术详解系列（二）" §2.1: a query built
    to give weights 0.05/0.10/0.70/0.15; the GPU must reproduce them and
    r = 0.05 h0 + 0.10 h1 + 0.70 h2 + 0.15 h3."""
    dev = device()
    note(f"worked example {dtype}")
    H, w, target = oracle_pins.worked_example_inputs(d=256, tokens=16, dtype=dtype)
    w32 = w.astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Hd = torch.from_numpy(H).to(dev).to(tdt)
    out, a = run(Hd, torch.from_numpy(w32).to(dev))
    tol = 1e-3 if dtype == "bf16" else 1e-5
    assert np.max(np.abs(host(a) - target)) <= tol
    expect = sum(c * H[i].astype(np.float64) for i, c in enumerate(target))
    r_ref, a_ref = oracle_aggregate(H, w32)
    compare(host(out), host(a), r_ref, a_ref, dtype == "bf16", f"worked example {dtype}")
    assert np.max(np.abs(host(out) - expect)) <= (1e-2 if dtype == "bf16" else 1e-5) * np.max(np.abs(expect))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_source_is_identity(dtype):
    dev = device()
    H = synth.sources(1, 300, 7168, seed=5, dtype=dtype, device=dev)
    out, a = run(H, synth.query(7168, seed=5, device=dev))
    assert torch.equal(out, H[0]) and bool(torch.all(a == 1.0))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_query_is_the_uniform_mixer(dtype):
    dev = device()
    S, T, d = 9, 50, 7168
    H = synth.sources(S, T, d, seed=6, dtype=dtype, device=dev)
    out, a = run(H, torch.zeros(d, device=dev))
    assert np.max(np.abs(host(a) - 1.0 / S)) <= 1e-7
    r_ref, a_ref = oracle_aggregate(host(H), np.zeros(d, np.float32))
    compare(host(out), host(a), r_ref, a_ref, dtype == "bf16", "zero query")
    np.testing.assert_allclose(r_ref, host(H).astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-12)


def test_identical_sources_and_zero_source_and_tiny_source():
    dev = device()
    S, T, d = 6, 40, 7168
    H = synth.sources(S, T, d, seed=7, dtype="bf16", device=dev)
    H[1] = H[0]
    H[2] = H[0]
    H[3].zero_()                       # all-zero source: logit 0, still weighted
    H[4].mul_(1e-4)                    # mean square comparable to eps
    w = synth.query(d, seed=7, device=dev)
    out, a = run(H, w)
    ha = host(a)
    assert np.max(np.abs(ha[:, 1] - ha[:, 0])) == 0 and np.max(np.abs(ha[:, 2] - ha[:, 0])) == 0
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    assert np.all(a_ref[:, 3] > 0)
    compare(host(out), ha, r_ref, a_ref, True, "identical / zero / tiny sources")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_huge_query_gives_one_hot_without_overflow(dtype):
    """Logits of order 1e4: the max subtraction keeps everything finite, and where
    the oracle is one-hot the GPU must be too (near-ties are ill-conditioned at
    this scale and are only checked for finiteness)."""
    dev = device()
    S, T, d = 9, 64, 7168
    H = synth.sources(S, T, d, seed=8, dtype=dtype, device=dev)
    w = synth.query(d, seed=8, device=dev) * 1e4
    out, a = run(H, w)
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    assert np.all(np.isfinite(host(a))) and np.all(np.isfinite(host(out)))
    clear = a_ref.max(axis=1) > 1 - 1e-9
    assert clear.sum() > T // 2
    compare(host(out)[clear], host(a)[clear], r_ref[clear], a_ref[clear], dtype == "bf16", "huge query")


def test_empty_batch_touches_nothing():
    dev = device()
    H = torch.empty((9, 0, 7168), dtype=torch.bfloat16, device=dev)
    out, a = run(H, torch.zeros(7168, device=dev))
    assert out.shape == (0, 7168) and a.shape == (0, 9)


def test_source_stride_larger_than_a_source():
    """Sources taken from a store sized for more tokens (stride > T*d)."""
    dev = device()
    S, T, Tcap, d = 9, 100, 133, 7168
    big = synth.sources(S, Tcap, d, seed=9, dtype="bf16", device=dev)
    H = big[:, :T]
    assert H.stride(0) == Tcap * d
    w = synth.query(d, seed=9, device=dev)
    out, a = run(H, w)
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(host(out), host(a), r_ref, a_ref, True, "strided sources")


def test_batch_beyond_the_grid_cap():
    """More tokens than one launch's grid holds (CUs x 4096): the host splits the
    batch over several launches of one workgroup per token, in XCD runs."""
    dev = device()
    S, T, d = 3, 256 * 4096 + 4099, 8
    cfg = B.aggregate_config(S, T, d, torch.bfloat16, torch.cuda.get_device_properties(dev).multi_processor_count)
    assert cfg["grid"] < T
    note(f"grid-stride T={T} grid={cfg['grid']}")
    H = synth.sources(S, T, d, seed=10, dtype="bf16", device=dev)
    w = synth.query(d, seed=10, device=dev)
    out, a = run(H, w)
    r_ref, a_ref = oracle_aggregate(host(H), host(w), chunk=1 << 16)
    compare(host(out), host(a), r_ref, a_ref, True, "grid-stride")


def test_weights_optional_and_side_stream():
    dev = device()
    S, T, d = 9, 77, 7168
    H = synth.sources(S, T, d, seed=11, dtype="bf16", device=dev)
    w = synth.query(d, seed=11, device=dev)
    ref_out, _ = run(H, w)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        out2, none = B.aggregate(H, w, want_weights=False)
    s.synchronize()
    assert none is None and torch.equal(out2, ref_out)


def test_bitwise_deterministic():
    dev = device()
    S, T, d = 9, 2048, 7168
    H = synth.sources(S, T, d, seed=12, dtype="bf16", device=dev)
    w = synth.query(d, seed=12, device=dev)
    o1, a1 = run(H, w)
    o2, a2 = run(H, w)
    assert torch.equal(o1, o2) and torch.equal(a1, a2)


def test_misaligned_and_aliased_buffers_raise():
    dev = device()
    H = synth.sources(2, 4, 64, seed=13, dtype="bf16", device=dev)
    w = synth.query(64, seed=13, device=dev)
    flat = torch.empty(4 * 64 + 8, dtype=torch.bfloat16, device=dev)
    with pytest.raises(B.AttnResError) as e:
        B.aggregate(H, w, out=flat[4:4 + 4 * 64])
    assert e.value.status == B.EUNSUPPORTED
    with pytest.raises(B.AttnResError) as e:
        B.aggregate(H, w, out=H[1].reshape(-1))
    assert e.value.status == B.EALIAS
