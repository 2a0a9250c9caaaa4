"""GPU parity of the split-row instance (decode-size batches: one 64-lane
workgroup per 1 KiB chunk of each token's row, partial sums exchanged through
the exchange workspace) against the oracle, and its bookkeeping: repeated calls
on one workspace, the fused update, batches past its limit, the timeout flag."""

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import synth
from oracle import attnres_oracle as orc
from tests.gpu_util import compare, device, host, note, oracle_aggregate

pytestmark = pytest.mark.gpu


def timeout_flag(x: torch.Tensor) -> int:
    """The workspace header's sticky flag (uint32 at byte 8): a chunk whose wait ran out."""
    return int(x[8:12].cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,T,d", [
    (1, 1, 7168), (9, 1, 7168), (9, 8, 7168), (9, 64, 7168), (4, 3, 7168), (2, 5, 7168),
    (5, 7, 264), (9, 2, 7176), (6, 256, 2048), (3, 9, 16384), (7, 4, 1000), (9, 1, 8),
])
def test_split_matches_oracle(dtype, S, T, d):
    dev = device()
    if dtype == "f32" and d > B.MAX_D_F32:
        pytest.skip("float32 rows are limited to MAX_D_F32")
    note(f"split aggregate {dtype} S={S} T={T} d={d}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=S * 17 + T, dtype=dtype, device=dev)
    w = synth.query(d, seed=T + 3, device=dev)
    x = B.new_exchange(T, d, tdt, dev)
    assert x is not None
    out, a = B.aggregate(H, w, exchange=x)
    torch.cuda.synchronize()
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(host(out), host(a), r_ref, a_ref, dtype == "bf16", f"split {dtype} S={S} T={T} d={d}")
    assert timeout_flag(x) == 0


@pytest.mark.parametrize("T", [1, 8, 64])
def test_split_repeated_calls_are_bitwise_reproducible(T):
    """The workspace keeps itself consistent across calls: the same inputs give
    the same bits call after call, with other shapes in between."""
    dev = device()
    d, S = 7168, 9
    note(f"split repeat T={T}")
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=T, device=dev)
    w = synth.query(d, seed=1, device=dev)
    x = B.new_exchange(256, d, torch.bfloat16, dev)       # sized for the largest batch, serves smaller ones
    first, a1 = B.aggregate(H, w, exchange=x)
    first, a1 = first.clone(), a1.clone()
    H2 = synth.sources(4, 3, d, seed=99, device=dev)
    for k in range(5):
        B.aggregate(H2, w, exchange=x)                   # another shape on the same workspace
        out, a = B.aggregate(H, w, exchange=x)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first.view(torch.int16)), f"call {k}"
        assert torch.equal(a.view(torch.int32), a1.view(torch.int32)), f"call {k}"
    # the generation advanced once per launch (header word 0), and no wait ran out
    assert int(x[0:4].cpu().numpy().view(np.uint32)[0]) == 11
    assert timeout_flag(x) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_completed,partial,finalize", [(0, False, False), (3, True, False), (6, True, True),
                                                          (7, True, False), (2, False, True)])
def test_split_fused_update_equals_the_pair(dtype, n_completed, partial, finalize):
    """attnres_accumulate_aggregate_ex in the split instance: the slot update is
    bit-exact (oracle accumulate) and the aggregation bit-identical to
    attnres_accumulate followed by attnres_aggregate_ex on the same workspace."""
    dev = device()
    T, d = 8, 7168
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    note(f"split fused {dtype} n={n_completed} partial={partial} finalize={finalize}")

    def fresh():
        st = B.SourceStore(T, d, dtype=tdt, device=dev)
        synth.sources(B.MAX_SOURCES, T, d, scale=(0.5, 50.0), seed=n_completed + 5, dtype=dtype,
                      out=st.slots)
        st.set_state(n_completed, partial)
        return st

    F = synth.layer_output(T, d, std=1.0, seed=7, tag=2, device=dev, dtype=dtype)
    w = synth.query(d, seed=11, device=dev)
    x = B.new_exchange(T, d, tdt, dev)
    st1 = fresh()
    slot = 1 + n_completed
    old = host(st1.slots[slot]).copy()
    out1, a1 = st1.accumulate_aggregate(F, finalize, w, exchange=x)
    st2 = fresh()
    st2.accumulate(F, finalize)
    out2, a2 = st2.aggregate(w, exchange=x)
    torch.cuda.synchronize()
    assert torch.equal(st1.slots.view(torch.int16 if dtype == "bf16" else torch.int32),
                       st2.slots.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(out1.view(torch.int16 if dtype == "bf16" else torch.int32),
                       out2.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(a1.view(torch.int32), a2.view(torch.int32))
    want = orc.accumulate(old if partial else None, host(F), dtype)
    assert np.array_equal(host(st1.slots[slot]).view(np.uint32), np.asarray(want, np.float32).view(np.uint32))
    r_ref, a_ref = oracle_aggregate(host(st1.sources()), host(w))
    compare(host(out1), host(a1), r_ref, a_ref, dtype == "bf16", f"split fused {dtype}")
    assert timeout_flag(x) == 0


def test_split_not_used_past_its_limit():
    """With a workspace, batches above SPLIT_MAX_TOKENS run the one-workgroup-per-
    token kernel: bit-identical to no workspace at all."""
    dev = device()
    T, d = B.SPLIT_MAX_TOKENS + 1, 1024
    H = synth.sources(9, T, d, seed=3, device=dev)
    w = synth.query(d, seed=4, device=dev)
    x = torch.zeros(B.exchange_bytes(B.SPLIT_MAX_TOKENS, d) + 4096, dtype=torch.uint8, device=dev)
    o1, a1 = B.aggregate(H, w, exchange=x)
    o2, a2 = B.aggregate(H, w)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(a1, a2)
    assert int(x[0:4].cpu().numpy().view(np.uint32)[0]) == 0     # the workspace was not touched


def test_split_on_a_side_stream():
    dev = device()
    T, d = 16, 7168
    H = synth.sources(9, T, d, seed=8, device=dev)
    w = synth.query(d, seed=9, device=dev)
    x = B.new_exchange(T, d, torch.bfloat16, dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out, a = B.aggregate(H, w, exchange=x)
    s.synchronize()
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(host(out), host(a), r_ref, a_ref, True, "split side stream")
