"""GPU parity of attnres_accumulate (bit-exact against the oracle) and of the
store's block bookkeeping, plus a full-compare depth schedule at a small size."""

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import schedule, synth
from oracle import attnres_oracle as orc
from tests.gpu_util import compare, device, host, note, oracle_aggregate, same_bits

pytestmark = pytest.mark.gpu


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,d", [(1, 8), (3, 7176), (257, 7168), (4099, 264)])
def test_accumulate_copy_then_add_is_bit_exact(dtype, T, d):
    dev = device()
    note(f"accumulate {dtype} T={T} d={d}")
    store = B.SourceStore(T, d, s_max=3, dtype=_tdt(dtype), device=dev)
    F1 = synth.layer_output(T, d, std=3.0, seed=T, tag=1, dtype=dtype, device=dev)
    F2 = synth.layer_output(T, d, std=0.01, seed=T, tag=2, dtype=dtype, device=dev)
    store.slots[2].fill_(7.0)                 # must stay untouched
    sentinel = store.slots[2].clone()
    store.accumulate(F1)                      # first layer of the block: copy
    torch.cuda.synchronize()
    assert torch.equal(store.slots[1], F1) and store.num_sources() == 2
    store.accumulate(F2, finalize_block=True)  # add, then close the block
    torch.cuda.synchronize()
    ref = orc.accumulate(host(F1), host(F2), dtype)
    assert same_bits(store.slots[1], ref)
    assert torch.equal(store.slots[2], sentinel)  # untouched
    assert store.n_completed == 1 and not store.partial_valid and store.num_sources() == 2


def test_accumulate_rounding_ties_and_wide_range():
    """bf16 sums that land on rounding ties and span many binades."""
    dev = device()
    T, d = 4, 4096
    rng = np.random.default_rng(0)
    p = orc.bf16_round((rng.normal(size=T * d) * np.exp(rng.uniform(-20, 20, T * d))).astype(np.float32))
    f = orc.bf16_round((rng.normal(size=T * d) * np.exp(rng.uniform(-20, 20, T * d))).astype(np.float32))
    # ties: 1 + 2^-8 (stays), 1 + 3*2^-8 (rounds up), negative mirror images
    ties = np.array([[1.0, 2.0 ** -8], [1.0 + 2.0 ** -7, 2.0 ** -8], [-1.0, -(2.0 ** -8)],
                     [-(1.0 + 2.0 ** -7), -(2.0 ** -8)], [256.0, 1.0], [257.0 + 1.0, 1.0]], np.float32)
    p[: len(ties)], f[: len(ties)] = ties[:, 0], ties[:, 1]
    store = B.SourceStore(T, d, s_max=2, dtype=torch.bfloat16, device=dev)
    pt = torch.from_numpy(p).view(T, d).to(dev).to(torch.bfloat16)
    ft = torch.from_numpy(f).view(T, d).to(dev).to(torch.bfloat16)
    store.accumulate(pt)
    store.accumulate(ft)
    torch.cuda.synchronize()
    assert same_bits(store.slots[1], orc.accumulate(p.reshape(T, d), f.reshape(T, d), "bf16"))


def test_empty_store_through_the_binding():
    """A store for T = 0 (its slots an empty tensor, whose pointer is null):
    updates and aggregations only advance the counters and return empty rows."""
    dev = device()
    d = 7168
    st = B.SourceStore(0, d, dtype=torch.bfloat16, device=dev)
    F = torch.empty((0, d), dtype=torch.bfloat16, device=dev)
    w = synth.query(d, seed=1, device=dev)
    st.accumulate(F)
    out, a = st.accumulate_aggregate(F, True, w)
    torch.cuda.synchronize()
    assert out.shape == (0, d) and a.shape[0] == 0
    assert (st.n_completed, st.partial_valid) == (1, 0)
    out, a = st.aggregate(w)
    assert out.shape == (0, d) and a.shape == (0, 2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,d", [(5, 7168), (129, 264), (1000, 7176), (3, 8)])
@pytest.mark.parametrize("state,finalize", [((0, 0), 0), ((0, 1), 0), ((2, 1), 1), ((3, 0), 1), ((7, 1), 0)])
def test_fused_update_aggregate_is_bit_identical_to_two_calls(dtype, T, d, state, finalize):
    """attnres_accumulate_aggregate == attnres_accumulate + attnres_aggregate:
    slot contents, residual, weights and bookkeeping, bit for bit."""
    dev = device()
    note(f"fused vs separate {dtype} T={T} d={d} state={state} finalize={finalize}")
    a_store = B.SourceStore(T, d, dtype=_tdt(dtype), device=dev)
    synth.sources(9, T, d, scale=(0.5, 50.0), seed=T + d, dtype=dtype, out=a_store.slots)
    b_store = B.SourceStore(T, d, dtype=_tdt(dtype), device=dev, slots=a_store.slots.clone())
    for st in (a_store, b_store):
        st.set_state(*state)
    F = synth.layer_output(T, d, std=2.0, seed=T, tag=3, dtype=dtype, device=dev)
    w = synth.query(d, seed=d, device=dev)
    a_store.accumulate(F, bool(finalize))
    out_a, wts_a = a_store.aggregate(w)
    out_b, wts_b = b_store.accumulate_aggregate(F, bool(finalize), w)
    torch.cuda.synchronize()
    assert (a_store.n_completed, a_store.partial_valid) == (b_store.n_completed, b_store.partial_valid)
    assert torch.equal(a_store.slots.view(torch.int16 if dtype == "bf16" else torch.int32),
                       b_store.slots.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(out_a.view(torch.int16 if dtype == "bf16" else torch.int32),
                       out_b.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(wts_a.view(torch.int32), wts_b.view(torch.int32))


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_schedule_matches_oracle_everywhere(dtype, fused):
    """30 layers in blocks of 4 (8 blocks, so up to 9 sources), ragged T and d,
    every layer's output and weights compared in full, block sums bit-exact."""
    dev = device()
    L, Bsz, T, d = 30, 4, 300, 520
    note(f"small schedule {dtype} fused={fused} L={L} block={Bsz} T={T} d={d}")
    store = B.SourceStore(T, d, dtype=_tdt(dtype), device=dev)
    synth.fill_normal_(store.h0, 1.0, seed=1, tag=1)
    Fs = [synth.layer_output(T, d, std=0.1, seed=1, tag=l, dtype=dtype, device=dev) for l in range(L)]
    Ws = [synth.query(d, seed=1, device=dev, tag=l) for l in range(L)]
    w_out = synth.query(d, seed=1, device=dev, tag=999)
    outs = torch.empty((L, T, d), dtype=_tdt(dtype), device=dev)
    wts = torch.zeros((L, T, 9), dtype=torch.float32, device=dev)
    final_r, final_a = schedule.run_schedule(store, Fs, Ws, Bsz, out=outs, weights=wts, final_query=w_out,
                                             fused=fused)
    torch.cuda.synchronize()
    ref = orc.run_schedule(host(store.h0), [host(F) for F in Fs], [host(w) for w in Ws], Bsz, dtype,
                           final_query=host(w_out))
    assert store.n_completed == 8 and ref["num_sources"][0] == 1
    for k, b in enumerate(ref["blocks"]):
        assert same_bits(store.slots[k + 1], b), f"block {k + 1}"
    for l in range(L):
        S = ref["num_sources"][l]
        a_gpu = host(wts[l]).reshape(-1)[: T * S].reshape(T, S)
        compare(host(outs[l]), a_gpu, ref["r"][l], ref["a"][l], dtype == "bf16", f"layer {l + 1} S={S}")
    compare(host(final_r), host(final_a), ref["final_r"], ref["final_a"], dtype == "bf16", "output layer")
    assert torch.equal(outs[0], store.h0)  # layer 1 sees only h_0
