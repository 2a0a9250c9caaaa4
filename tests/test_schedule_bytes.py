"""The algorithmic bytes the bench reports for the 93-layer schedule
(``workloads.Schedule.step_bytes``, a closed form by layer and block) against
an independent count: the schedule driver itself runs on a store that launches
nothing and instead adds up what each launch reads and writes, from what that
launch does (rows in and out, logits, weights, queries).  CPU only."""

import pytest
import torch

from depth_wise_attention_block_amd import schedule, workloads


class CountingStore:
    """The SourceStore interface the schedule driver uses, keeping the store
    state and counting each launch's HBM bytes instead of launching."""

    def __init__(self, T, d):
        self.T, self.d = T, d
        self.slots = torch.zeros((9, T, d), dtype=torch.bfloat16)
        self.n_completed, self.partial_valid = 0, False
        self.bytes = 0
        self.row = 2 * T * d                       # one bf16 row of every token

    def num_sources(self):
        return 1 + self.n_completed + int(self.partial_valid)

    def sources(self):
        return self.slots[: self.num_sources()]

    def _add_layer(self, finalize):
        self.partial_valid = True
        if finalize:
            self.n_completed, self.partial_valid = self.n_completed + 1, False

    def accumulate(self, layer_out, finalize_block=False, stream=None):
        # the layer output (and the old partial when adding) in, the slot out
        self.bytes += (2 if self.partial_valid else 1) * self.row + self.row
        self._add_layer(finalize_block)

    def accumulate_aggregate(self, layer_out, finalize_block, w, out=None, weights=None, *, want_weights=True,
                             eps=1e-5, stream=None):
        had_partial = self.partial_valid
        self._add_layer(finalize_block)
        S, T, d = self.num_sources(), self.T, self.d
        reads = (S - 1) * self.row + self.row + (self.row if had_partial else 0) + 4 * d
        writes = 2 * self.row + (4 * T * S if weights is not None else 0)
        self.bytes += reads + writes
        return out, weights

    def block_prepare(self, layer_out, close_block, w_split, inter, logits, weights0=None, *, eps=1e-5, stream=None):
        T, d = self.T, self.d
        had_partial = self.partial_valid
        complete_before = 1 + self.n_completed    # h_0 and the blocks already closed
        if close_block:
            self._add_layer(True)
        K, B = 1 + self.n_completed, inter.shape[0]
        reads = complete_before * self.row + B * 4 * d            # rows, prepared queries (bf16 hi + lo)
        if close_block:
            reads += self.row + (self.row if had_partial else 0)   # layer output, old partial
        writes = (self.row if close_block else 0) + B * self.row + 4 * B * T * K
        writes += 4 * T * K if weights0 is not None else 0
        self.bytes += reads + writes

    def block_merge(self, layer_out, w, inter, logits, out=None, weights=None, *, want_weights=True, eps=1e-5,
                    stream=None):
        T, d = self.T, self.d
        had_partial = self.partial_valid
        K = 1 + self.n_completed
        self._add_layer(False)
        reads = 2 * self.row + (self.row if had_partial else 0) + 4 * T * K + 4 * d   # R, F, old partial, logits, w
        writes = 2 * self.row + (4 * T * (K + 1) if weights is not None else 0)       # partial, residual, weights
        self.bytes += reads + writes
        return out, weights


def _run(mode, T=3, d=16, layers=93, block_size=12, two_phase_from=3):
    store = CountingStore(T, d)

    def counting_aggregate(sources, w, out=None, weights=None, *, want_weights=True, eps=1e-5, stream=None):
        S = sources.shape[0]
        store.bytes += S * store.row + store.row + (4 * T * S if weights is not None else 0) + 4 * d
        return out, weights

    F = [torch.zeros((T, d), dtype=torch.bfloat16) for _ in range(layers)]
    W = [torch.zeros(d) for _ in range(layers)]
    kw = {}
    if mode == "two_phase":
        nblocks = (layers + block_size - 1) // block_size
        kw = dict(two_phase_from=two_phase_from, inter=torch.zeros((block_size, T, d), dtype=torch.bfloat16),
                  logits=torch.zeros(block_size * T * 8), queries_split=[torch.zeros((3, 1)) for _ in range(nblocks)])
    saved = schedule.aggregate
    schedule.aggregate = counting_aggregate
    try:
        schedule.run_schedule(store, F, W, block_size, out=torch.zeros((T, d), dtype=torch.bfloat16),
                              weights=torch.zeros((T, 9)), final_query=torch.zeros(d),
                              final_out=torch.zeros((T, d), dtype=torch.bfloat16), final_weights=torch.zeros((T, 9)),
                              fused=mode != "unfused", **kw)
    finally:
        schedule.aggregate = saved
    return store.bytes


@pytest.mark.parametrize("mode", ["unfused", "fused", "two_phase"])
@pytest.mark.parametrize("T,d", [(1, 8), (3, 16), (5, 24)])
def test_schedule_step_bytes_match_a_launch_by_launch_count(mode, T, d):
    """Equal at three shapes: every term of both counts is linear in T*d, T or
    d, so they are equal at the bench's T = 32768, d = 7168 too."""
    stub = object.__new__(workloads.Schedule)   # the closed form needs only the shape
    stub.T, stub.d, stub.layers, stub.block_size = T, d, 93, 12
    assert _run(mode, T=T, d=d) == workloads.Schedule.step_bytes(stub, mode)


def _run_backward(T, d, defer, layers=93, block_size=12):
    """The backward driver over a store in the forward's end state, with the
    three entry points it calls replaced by counters of their launches' bytes."""
    from depth_wise_attention_block_amd import binding

    nblocks = (layers + block_size - 1) // block_size
    store = CountingStore(T, d)
    store.n_completed, store.partial_valid = nblocks, False
    row2, row4 = 2 * T * d, 4 * T * d
    total = [0]

    def count_aggregate_backward(sources, w, grad_out, grad_sources, *, last_source=None, accumulate=0, defer=0,
                                 coef=None, coef_stride=0, grad_w=None, grad_last=None, workspace=None,
                                 form_dw=True, eps=1e-5, stream=None):
        S = grad_sources.shape[0]
        b = S * row2 + row2 + 4 * d                         # sources, dL/dr, query
        b += 4 * d if form_dw else 0                        # dL/dw out
        for s in range(S):
            if (defer >> s) & 1 or not form_dw:
                b += 12 * T                                    # three coefficients per token
            if not (defer >> s) & 1:
                b += row4 + (row4 if (accumulate >> s) & 1 else 0)   # the gradient row written (and read)
        if grad_last is not None:
            b += row2
        total[0] += b
        return grad_w

    def count_block_backward(sources, grad_outs, queries, coef, grad_sources, grad_ws, *, accumulate=0,
                             grad_last=None, coef_layer_stride=0, workspace=None, stream=None):
        n, B = sources.shape[0], len(grad_outs)
        b = n * row2 + B * row2 + 12 * n * B * T           # sources, dL/dr rows, coefficients
        b += sum(row4 + (row4 if (accumulate >> s) & 1 else 0) for s in range(n))   # gradient rows
        b += B * (4 * d + 8 * d)                           # each layer's query in; its dL/dw read and written
        if grad_last is not None:
            b += row2
        total[0] += b

    def count_partial_sums(layer_outs, out, stream=None):
        total[0] += 2 * len(layer_outs) * row2              # each layer output in, each partial sum out
        return out

    def count_partial_dw(rows, coef, coef_stride, coef_layer_stride, grad_ws, *, workspace=None, stream=None):
        # one coefficient per token of each given row in (the row itself is a
        # second read, as in the block's contraction), every dL/dw row out
        total[0] += sum(4 * T for r in rows if r is not None) + 4 * d * len(grad_ws)

    saved = binding.aggregate_backward, binding.block_backward, binding.partial_sums, binding.partial_dw
    binding.aggregate_backward, binding.block_backward, binding.partial_sums, binding.partial_dw = (
        count_aggregate_backward, count_block_backward, count_partial_sums, count_partial_dw)
    try:
        F = [torch.zeros((T, d), dtype=torch.bfloat16) for _ in range(layers)]
        W = [torch.zeros(d) for _ in range(layers)]
        G = [torch.zeros((T, d), dtype=torch.bfloat16) for _ in range(layers)]
        schedule.run_schedule_backward(store, F, W, block_size, G, final_query=torch.zeros(d),
                                       grad_final=torch.zeros((T, d), dtype=torch.bfloat16), defer=defer)
    finally:
        binding.aggregate_backward, binding.block_backward, binding.partial_sums, binding.partial_dw = saved
    return total[0]


@pytest.mark.parametrize("defer", [True, False], ids=["deferred", "per_layer"])
@pytest.mark.parametrize("T,d", [(1, 8), (3, 16), (5, 24)])
def test_backward_step_bytes_match_a_launch_by_launch_count(defer, T, d):
    stub = object.__new__(workloads.ScheduleBackward)
    stub.T, stub.d, stub.layers, stub.block_size = T, d, 93, 12
    assert _run_backward(T, d, defer) == workloads.ScheduleBackward.step_bytes(stub, defer)
