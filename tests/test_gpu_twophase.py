"""GPU parity of the two-phase schedule (kimi.papertok.ai ch. 4 §4.4, §4.6):
attnres_block_prepare (one pass over a block's inter-block sources for all its
queries) and attnres_block_merge (online-softmax merge of the partial), alone
and inside the depth schedule, against the oracle's plain definition."""

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import binding as B
from depth_wise_attention_block_amd import schedule, synth, workloads
from oracle import attnres_oracle as orc
from tests.gpu_util import compare, device, host, note, oracle_aggregate, same_bits, weighted_abs

pytestmark = pytest.mark.gpu


def test_split_queries_is_round_to_nearest_hi_then_lo():
    dev = device()
    w = synth.query(7176, seed=4, device=dev).view(1, -1).repeat(3, 1) * torch.tensor([[1.0], [1e-3], [37.0]],
                                                                                     device=dev)
    w = w.contiguous()
    ws = B.split_queries(w)
    torch.cuda.synchronize()
    assert tuple(ws.shape) == (1, 2, 7176 // 8, 4, 8)
    rows = B.unpack_prepared_queries(ws, 4)
    hw = host(w)
    hi = orc.bf16_round(hw)
    lo = orc.bf16_round((hw - hi).astype(np.float32))
    assert same_bits(rows[:3, 0], hi) and same_bits(rows[:3, 1], lo)
    assert not rows[3].any(), "the group's padding query is zero"


def _store(T, d, seed, n_completed, partial_valid, dev):
    st = B.SourceStore(T, d, dtype=torch.bfloat16, device=dev)
    synth.sources(9, T, d, scale=(0.5, 50.0), seed=seed, out=st.slots)
    st.set_state(n_completed, partial_valid)
    return st


@pytest.mark.parametrize("T,d", [(37, 7168), (5, 264), (300, 7176)])
@pytest.mark.parametrize("n_completed,partial_valid,close", [(0, False, False), (3, False, False), (6, True, True),
                                                            (4, False, True), (7, False, False),
                                                            (2, True, True), (1, False, True)])
@pytest.mark.parametrize("Bq", [1, 12, 16])
def test_prepare_matches_oracle(T, d, n_completed, partial_valid, close, Bq):
    dev = device()
    note(f"prepare T={T} d={d} n={n_completed} partial={partial_valid} close={close} B={Bq}")
    st = _store(T, d, T + d + n_completed, n_completed, partial_valid, dev)
    F = synth.layer_output(T, d, std=1.0, seed=T, tag=5, device=dev)
    slots_before = host(st.slots)
    K = 1 + n_completed + (1 if close else 0)
    W = torch.stack([synth.query(d, seed=b, device=dev, tag=b) for b in range(Bq)])
    inter = torch.empty((Bq, T, d), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((Bq, T, K), dtype=torch.float32, device=dev)
    w0 = torch.empty((T, K), dtype=torch.float32, device=dev)
    st.block_prepare(F if close else None, close, B.split_queries(W), inter, logits, w0)
    torch.cuda.synchronize()
    assert st.n_completed == K - 1 and not st.partial_valid
    H = slots_before[:K].copy()
    if close:
        slot = K - 1
        H[slot] = orc.accumulate(slots_before[slot] if partial_valid else None, host(F), "bf16")
        assert same_bits(st.slots[slot], H[slot]), "closed block representation"
    for b in range(Bq):
        r_ref, a_ref = oracle_aggregate(H, host(W[b]))
        a_gpu = torch.softmax(logits[b].double(), dim=1).cpu().numpy()
        compare(host(inter[b]), a_gpu, r_ref, a_ref, True, f"prepare query {b}")
        if b == 0:
            assert np.max(np.abs(host(w0) - a_ref)) <= 1e-3


def test_prepare_split_over_launches_beyond_the_grid_cap():
    """More tokens than one launch's grid (CUs x 4096): the host splits the
    inter-block pass over several launches of one workgroup per token.  Tokens
    on both sides of the launch boundary, the ends and a random sample match the
    oracle, and the closed block is written at every one of them."""
    dev = device()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    cap = cus * 4096
    T, d, n_completed, Bq = cap + 4099, 8, 2, 5
    note(f"prepare over launches T={T} cap={cap}")
    st = _store(T, d, 21, n_completed, True, dev)
    F = synth.layer_output(T, d, std=1.0, seed=21, tag=5, device=dev)
    K = n_completed + 2
    idx = torch.unique(torch.cat([synth.token_sample(T, 256, 4, seed=21), torch.arange(cap - 3, cap + 3)]))
    idx_dev = idx.to(dev)
    before = host(st.slots[:K].index_select(1, idx_dev))
    W = torch.stack([synth.query(d, seed=b, device=dev, tag=b) for b in range(Bq)])
    inter = torch.empty((Bq, T, d), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((Bq, T, K), dtype=torch.float32, device=dev)
    st.block_prepare(F, True, B.split_queries(W), inter, logits)
    torch.cuda.synchronize()
    H = before.copy()
    H[K - 1] = orc.accumulate(before[K - 1], host(F.index_select(0, idx_dev)), "bf16")
    assert same_bits(st.slots[K - 1].index_select(0, idx_dev), H[K - 1]), "closed block representation"
    for b in range(Bq):
        r_ref, a_ref = oracle_aggregate(H, host(W[b]))
        a_gpu = torch.softmax(logits[b].index_select(0, idx_dev).double(), dim=1).cpu().numpy()
        compare(host(inter[b].index_select(0, idx_dev)), a_gpu, r_ref, a_ref, True, f"prepare over launches, query {b}")
    del st, inter, logits
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,d", [(64, 7168), (9, 520)])
def test_merge_matches_oracle_through_a_block(T, d):
    """One block of 12 layers at K = 6 inter-block sources: prepare, then 11
    merges, each compared with the plain aggregation over all its sources."""
    dev = device()
    K, Bq = 6, 12
    st = _store(T, d, 11, K - 1, False, dev)
    H = host(st.slots[:K])
    W = torch.stack([synth.query(d, seed=b, device=dev, tag=40 + b) for b in range(Bq)])
    Fs = [synth.layer_output(T, d, std=0.3, seed=b, tag=50 + b, device=dev) for b in range(Bq)]
    inter = torch.empty((Bq, T, d), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((Bq, T, K), dtype=torch.float32, device=dev)
    st.block_prepare(None, False, B.split_queries(W), inter, logits)
    partial = None
    for i in range(2, Bq + 1):
        note(f"merge layer {i} T={T} d={d}")
        out, wts = st.block_merge(Fs[i - 2], W[i - 1], inter[i - 1], logits[i - 1])
        torch.cuda.synchronize()
        partial = orc.accumulate(partial, host(Fs[i - 2]), "bf16")
        assert same_bits(st.slots[K], partial), f"partial after layer {i - 1}"
        Hi = np.concatenate([H, partial[None]], axis=0)
        r_ref, a_ref = oracle_aggregate(Hi, host(W[i - 1]))
        compare(host(out), host(wts), r_ref, a_ref, True, f"merge layer {i}",
                extra_rounding=weighted_abs(Hi, a_ref, K))


@pytest.mark.parametrize("add", [False, True])
def test_merge_forms_bit_identical(add):
    """Small batches take the per-token merge (every load of a token issued up
    front), larger ones the looping form; the arithmetic is the same, so the
    first 500 tokens of a 600-token merge (looping form) equal a 500-token
    merge of the same rows (per-token form) bit for bit, in the partial slot,
    the residual and the weights."""
    dev = device()
    d, K = 7168, 5
    big, small = 600, 500
    st = _store(big, d, 31, K - 1, add, dev)   # K inter-block sources; the partial is slot K
    W = synth.query(d, seed=3, device=dev, tag=70)
    F = synth.layer_output(big, d, std=0.3, seed=3, tag=71, device=dev)
    inter = synth.layer_output(big, d, std=1.0, seed=3, tag=72, device=dev)
    logits = torch.randn((big, K), generator=torch.Generator(device=dev).manual_seed(5), device=dev)
    st_s = B.SourceStore(small, d, dtype=torch.bfloat16, device=dev,
                         slots=st.slots[:, :small].contiguous())
    st_s.set_state(st.n_completed, st.partial_valid)
    note(f"merge forms add={add}: T={big} (looping) and T={small} (per token)")
    out_b, w_b = st.block_merge(F, W, inter, logits)
    out_s, w_s = st_s.block_merge(F[:small].contiguous(), W, inter[:small].contiguous(), logits[:small].contiguous())
    torch.cuda.synchronize()
    assert same_bits(st.slots[K, :small], host(st_s.slots[K])), "partial slot"
    assert same_bits(out_b[:small], host(out_s)), "residual"
    assert same_bits(w_b[:small], host(w_s)), "weights"


def test_merge_in_place_over_the_inter_row():
    dev = device()
    T, d, K = 33, 7168, 4
    st = _store(T, d, 12, K - 1, False, dev)
    W = torch.stack([synth.query(d, seed=b, device=dev, tag=60 + b) for b in range(2)])
    inter = torch.empty((2, T, d), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((2, T, K), dtype=torch.float32, device=dev)
    st.block_prepare(None, False, B.split_queries(W), inter, logits)
    ref_store = B.SourceStore(T, d, dtype=torch.bfloat16, device=dev, slots=st.slots.clone())
    ref_store.set_state(st.n_completed, st.partial_valid)
    F = synth.layer_output(T, d, std=1.0, seed=3, tag=61, device=dev)
    separate, wa = ref_store.block_merge(F, W[1], inter[1], logits[1])
    torch.cuda.synchronize()
    separate = separate.clone()
    same, wb = st.block_merge(F, W[1], inter[1], logits[1], out=inter[1])
    torch.cuda.synchronize()
    assert same.data_ptr() == inter[1].data_ptr()
    assert torch.equal(same.view(torch.int16), separate.view(torch.int16)) and torch.equal(wa, wb)


def _check_schedule(L, Bsz, T, d, two_phase_from, out3d, tag):
    """Every layer of an L-layer schedule in blocks of Bsz against the oracle."""
    dev = device()
    note(f"{tag}: L={L} block={Bsz} T={T} d={d} two-phase from {two_phase_from} out3d={out3d}")
    store = B.SourceStore(T, d, dtype=torch.bfloat16, device=dev)
    synth.fill_normal_(store.h0, 1.0, seed=1, tag=1)
    Fs = [synth.layer_output(T, d, std=0.1, seed=1, tag=l, device=dev) for l in range(L)]
    Ws = [synth.query(d, seed=1, device=dev, tag=l) for l in range(L)]
    w_out = synth.query(d, seed=1, device=dev, tag=999)
    got_r, got_a = [], []
    outs = torch.empty((L, T, d), dtype=torch.bfloat16, device=dev) if out3d else None
    wts = torch.zeros((T, 9), dtype=torch.float32, device=dev)

    def grab(l, r, a):
        got_r.append(host(r))
        got_a.append(host(a))

    final_r, final_a = schedule.run_schedule(store, Fs, Ws, Bsz, out=outs, weights=wts, final_query=w_out,
                                             on_layer=grab, two_phase_from=two_phase_from)
    torch.cuda.synchronize()
    ref = orc.run_schedule(host(store.h0), [host(F) for F in Fs], [host(w) for w in Ws], Bsz, "bf16",
                           final_query=host(w_out))
    for k, b in enumerate(ref["blocks"]):
        assert same_bits(store.slots[k + 1], b), f"block {k + 1}"
    # rebuild each layer's sources to size the extra rounding of the inter part
    blocks = ref["blocks"]
    first_two_phase = two_phase_from if two_phase_from is not None else L + 1
    for l in range(1, L + 1):
        n, i = (l - 1) // Bsz + 1, (l - 1) % Bsz + 1
        srcs = [host(store.h0)] + blocks[:n - 1]
        if i >= 2:
            part = None
            for j in range((n - 1) * Bsz + 1, l):
                part = orc.accumulate(part, host(Fs[j - 1]), "bf16")
            srcs.append(part)
        Hs = np.stack(srcs)
        extra = weighted_abs(Hs, ref["a"][l - 1], n) if (n >= first_two_phase and i >= 2) else None
        compare(got_r[l - 1], got_a[l - 1], ref["r"][l - 1], ref["a"][l - 1], True, f"layer {l} S={len(srcs)}",
                extra_rounding=extra)
    compare(host(final_r), host(final_a), ref["final_r"], ref["final_a"], True, "output layer")


def _random_schedules(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        bsz = int(rng.integers(1, 21))
        nblocks = int(rng.integers(1, 9))
        L = int(rng.integers((nblocks - 1) * bsz + 1, nblocks * bsz + 1))
        tpf = None if rng.random() < 0.3 else int(rng.integers(1, nblocks + 1))
        out.append((L, bsz, int(rng.integers(1, 100)), int(8 * rng.integers(1, 257)), tpf, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("case", _random_schedules(6, 31), ids=lambda c: f"L{c[0]}-b{c[1]}-T{c[2]}-d{c[3]}-from{c[4]}")
def test_random_schedules_match_oracle(case):
    """Seeded random layer counts, block sizes (1-20: more than 16 layers per
    block takes two inter-block passes), up to 8 blocks, ragged T and d, and
    the two-phase schedule from a random block (or not at all)."""
    L, bsz, T, d, tpf, out3d = case
    _check_schedule(L, bsz, T, d, tpf, out3d, "random schedule")


@pytest.mark.parametrize("two_phase_from", [1, 2, 4])
@pytest.mark.parametrize("out3d", [True, False])
def test_small_schedule_two_phase_matches_oracle(two_phase_from, out3d):
    """30 layers in blocks of 4 (8 blocks, up to 9 sources), every layer compared."""
    _check_schedule(30, 4, 300, 520, two_phase_from, out3d, "two-phase schedule")


@pytest.mark.parametrize("two_phase_from", [1, None])
def test_sublayer_granularity_schedule(two_phase_from):
    """One aggregation per residual sublayer (attention and MLP each with its own
    query), as in the reduced mechanism probe of llm-atlas.k1412.top/k3
    (16 transformer blocks, 32 residual sublayers): 20 layers = 40 sublayer
    steps in blocks of 10 layers = 20 steps.  Two-phase blocks then hold 20
    queries, more than one inter-block pass takes: the schedule runs two passes
    per block, the first closing the previous block."""
    _check_schedule(40, 20, 96, 264, two_phase_from, False, "sublayer schedule")


def test_schedule_93_two_phase_sampled():
    """Full-size 93-layer schedule, T = 32768, two-phase from block 3 (the bench's
    configuration), checked at sampled tokens through every layer."""
    dev = device()
    cfg = synth.WORKLOADS["schedule_93"]
    T = cfg["T"]
    note(f"two-phase schedule T={T}")
    wl = workloads.Schedule(T, layers=cfg["layers"], block_size=cfg["block_size"], seed=0, device=dev,
                            h0_scale=cfg["h0_scale"], layer_out_std=cfg["layer_out_std"])
    rows = synth.token_sample(T, 192, 32, seed=2)
    idx = rows.to(dev)
    got_r, got_a = [], []

    def grab(l, r, a):
        got_r.append(host(r.index_select(0, idx)))
        got_a.append(host(a.index_select(0, idx)))

    wl.step(on_layer=grab, mode="two_phase")
    torch.cuda.synchronize()
    hsel = host(wl.store.h0.index_select(0, idx))
    Fsel = [host(F.index_select(0, idx)) for F in wl.F]
    ref = orc.run_schedule(hsel, Fsel, [host(w) for w in wl.W], cfg["block_size"], "bf16",
                           final_query=host(wl.w_out))
    for k, b in enumerate(ref["blocks"]):
        assert same_bits(wl.store.slots[k + 1].index_select(0, idx), b), f"block {k + 1}"
    Bsz = cfg["block_size"]
    for l in range(1, cfg["layers"] + 1):
        n, i = (l - 1) // Bsz + 1, (l - 1) % Bsz + 1
        extra = None
        if n >= workloads.Schedule.TWO_PHASE_FROM and i >= 2:
            Hs = np.stack([hsel] + ref["blocks"][:n - 1])
            extra = weighted_abs(Hs, ref["a"][l - 1], n)
        compare(got_r[l - 1], got_a[l - 1], ref["r"][l - 1], ref["a"][l - 1], True, f"layer {l}",
                extra_rounding=extra)
    compare(host(wl.final_out.index_select(0, idx)), host(wl.final_weights.index_select(0, idx)),
            ref["final_r"], ref["final_a"], True, "output layer")
    del wl
    torch.cuda.empty_cache()
