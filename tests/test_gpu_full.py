"""GPU parity beyond 9 sources: the batched online-softmax path of
attnres_aggregate, and the Full AttnRes schedule (every earlier layer output is
a source; kimi.papertok.ai ch. 4 §4.2)."""

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import schedule, synth
from oracle import attnres_oracle as orc
from tests.gpu_util import compare, device, host, note, oracle_aggregate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,T,d", [(10, 33, 7168), (17, 5, 264), (18, 64, 7176), (94, 37, 7168),
                                   (130, 3, 2048), (256, 2, 520)])
def test_many_sources_match_oracle(dtype, S, T, d):
    dev = device()
    note(f"many sources {dtype} S={S} T={T} d={d}")
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=S + T, dtype=dtype, device=dev)
    w = synth.query(d, seed=S, device=dev)
    out, a = B.aggregate(H, w)
    torch.cuda.synchronize()
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(host(out), host(a), r_ref, a_ref, dtype == "bf16", f"{dtype} S={S} T={T} d={d}")


def test_many_sources_closed_forms():
    """Zero query -> 1/S and the mean; a huge query -> one-hot without overflow,
    with the winner in a late batch."""
    dev = device()
    S, T, d = 40, 16, 7168
    H = synth.sources(S, T, d, seed=3, device=dev)
    out, a = B.aggregate(H, torch.zeros(d, device=dev))
    torch.cuda.synchronize()
    assert np.max(np.abs(host(a) - 1.0 / S)) <= 1e-7
    w = synth.query(d, seed=4, device=dev) * 1e4
    out, a = B.aggregate(H, w)
    torch.cuda.synchronize()
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    assert np.all(np.isfinite(host(a))) and np.all(np.isfinite(host(out)))
    clear = a_ref.max(axis=1) > 1 - 1e-9
    assert clear.sum() > T // 2 and np.any(np.argmax(a_ref, 1) >= 9)
    compare(host(out)[clear], host(a)[clear], r_ref[clear], a_ref[clear], True, "huge query, 40 sources")


def test_many_sources_grid_stride_and_determinism():
    dev = device()
    S, T, d = 12, 256 * 4096 + 77, 8
    H = synth.sources(S, T, d, seed=5, device=dev)
    w = synth.query(d, seed=5, device=dev)
    o1, a1 = B.aggregate(H, w)
    o2, a2 = B.aggregate(H, w)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(a1, a2)
    rows = synth.token_sample(T, 2048, 64, seed=5)
    idx = rows.to(dev)
    r_ref, a_ref = oracle_aggregate(host(H.index_select(1, idx)), host(w))
    compare(host(o1.index_select(0, idx)), host(a1.index_select(0, idx)), r_ref, a_ref, True, "12 sources, T>grid")


def test_many_sources_xcd_runs_with_a_ragged_tail():
    """From 4,096 tokens on each XCD takes runs of 32 consecutive tokens; a
    batch that is no multiple of 8 runs leaves the last run partly empty."""
    dev = device()
    S, T, d = 20, 4096 + 37, 7168
    cfg = B.aggregate_config(S, T, d, torch.bfloat16, torch.cuda.get_device_properties(dev).multi_processor_count)
    assert cfg["xcd_run"] == 32
    note(f"many sources, XCD runs, S={S} T={T} d={d}")
    H = synth.sources(S, T, d, seed=6, device=dev)
    w = synth.query(d, seed=6, device=dev)
    out, a = B.aggregate(H, w)
    torch.cuda.synchronize()
    idx = synth.token_sample(T, 512, 64, seed=6).to(dev)
    r_ref, a_ref = oracle_aggregate(host(H.index_select(1, idx)), host(w))
    compare(host(out.index_select(0, idx)), host(a.index_select(0, idx)), r_ref, a_ref, True, "20 sources, runs")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_full_attnres_schedule_matches_oracle(dtype):
    """93 layers, each aggregating h_0 and all earlier outputs (S = 1..93), plus
    the output layer over 94 rows."""
    dev = device()
    L, T, d = 93, 40, 264
    note(f"full attnres schedule {dtype} L={L} T={T} d={d}")
    rows = torch.empty((L + 1, T, d), dtype=synth.torch_dtype(dtype), device=dev)
    synth.fill_normal_(rows[0], 1.0, seed=7, tag=1)
    for l in range(1, L + 1):
        synth.layer_output(T, d, std=0.5, seed=7, tag=l, dtype=dtype, device=dev, out=rows[l])
    Ws = [synth.query(d, seed=7, device=dev, tag=l) for l in range(L)]
    w_out = synth.query(d, seed=7, device=dev, tag=999)
    outs = torch.empty((L, T, d), dtype=rows.dtype, device=dev)
    wts = torch.zeros((L, T, L + 1), dtype=torch.float32, device=dev)
    final_r, final_a = schedule.run_full_schedule(rows, Ws, out=outs, weights=wts, final_query=w_out)
    torch.cuda.synchronize()
    per_layer, final = orc.run_full_schedule(host(rows[0]), [host(rows[l]) for l in range(1, L + 1)],
                                             [host(w) for w in Ws], final_query=host(w_out))
    for l in range(L):
        a_gpu = host(wts[l]).reshape(-1)[: T * (l + 1)].reshape(T, l + 1)
        compare(host(outs[l]), a_gpu, per_layer[l][0], per_layer[l][1], dtype == "bf16", f"full layer {l + 1}")
    compare(host(final_r), host(final_a), final[0], final[1], dtype == "bf16", "full output layer (94 sources)")
