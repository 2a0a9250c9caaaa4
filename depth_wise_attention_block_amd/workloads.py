"""Synthetic workloads and their steps, shared by the bench and the parity tests
so both time and check exactly the same launches.

* ``LayerStep``: one layer of the hot path at S = 9 -- the store holds h_0,
  seven completed block representations and the current block's partial sum
  (K3's last block: kimi.papertok.ai ch. 4 §4.5); a step adds the previous
  layer's output into the partial (read-modify-write) and aggregates the nine
  sources -- one ``attnres_accumulate_aggregate`` launch, or (``fused=False``)
  ``attnres_accumulate`` then ``attnres_aggregate``.  Used at T = 4096 (single
  layer), T in {1, 8, 64, 256} (decode batches) and T = 262144 (long-context
  prefill chunk).
* ``Schedule``: the whole 93-layer depth path at one batch of tokens -- every
  layer's aggregation and partial-sum update with block closing every 12
  layers, then the output layer's aggregation over h_0 and the 8 block
  representations (per layer, fused, or two-phase from block 3).
* ``ManySources``: one Full AttnRes aggregation over many sources.
* ``LayerBackward``: the backward of one 9-source aggregation.
* ``ScheduleBackward``: the whole 93-layer depth path in reverse -- the output
  layer, then every layer with each block's partial sums recomputed and its
  inter-block gradients deferred to one pass per block.

Each class gives ``step`` and ``step_bytes`` (the algorithmic HBM bytes of a
step).  Inputs come from :mod:`.synth` (seeded, generated on the device).
"""

from __future__ import annotations

import torch

from . import synth
from .binding import MAX_SOURCES, SourceStore
from .schedule import block_queries_split, closes_block, run_schedule


class LayerStep:
    def __init__(self, T: int, d: int = 7168, *, seed: int = 0, device="cuda", scale=(0.5, 50.0),
                 layer_out_std: float = 1.0):
        self.T, self.d = T, d
        self.store = SourceStore(T, d, s_max=MAX_SOURCES, dtype=torch.bfloat16, device=device)
        synth.sources(MAX_SOURCES, T, d, scale=scale, seed=seed, out=self.store.slots)
        self.store.set_state(MAX_SOURCES - 2, True)   # h0, b1..b7, partial
        self.F = synth.layer_output(T, d, std=layer_out_std, seed=seed, tag=1, device=device)
        self.w = synth.query(d, seed=seed, device=device)
        self.out = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.weights = torch.empty((T, MAX_SOURCES), dtype=torch.float32, device=device)

    def accumulate(self):
        self.store.accumulate(self.F, finalize_block=False)

    def aggregate(self):
        self.store.aggregate(self.w, self.out, self.weights)

    def fused(self):
        self.store.accumulate_aggregate(self.F, False, self.w, self.out, self.weights)

    def step(self, fused: bool = True):
        if fused:
            self.fused()
        else:
            self.accumulate()
            self.aggregate()

    # Algorithmic HBM bytes (each stream read or written once).
    def aggregate_bytes(self) -> int:
        S, T, d = MAX_SOURCES, self.T, self.d
        return T * (2 * S * d + 2 * d + 4 * S) + 4 * d

    def accumulate_bytes(self) -> int:
        return 3 * 2 * self.T * self.d

    def fused_bytes(self) -> int:
        """One fused launch: 8 untouched sources + old partial + layer output in,
        new partial + residual + weights out."""
        S, T, d = MAX_SOURCES, self.T, self.d
        return T * (2 * (S + 1) * d + 2 * 2 * d + 4 * S) + 4 * d

    def step_bytes(self, fused: bool = True) -> int:
        return self.fused_bytes() if fused else self.aggregate_bytes() + self.accumulate_bytes()


class Schedule:
    #: two-phase blocks start here: block n's one pass reads n inter-block rows
    #: and writes 12, which beats 12 one-pass layers from about n = 3 on
    TWO_PHASE_FROM = 3

    def __init__(self, T: int, d: int = 7168, *, layers: int = 93, block_size: int = 12, seed: int = 0,
                 device="cuda", h0_scale: float = 1.0, layer_out_std: float = 0.1):
        self.T, self.d, self.layers, self.block_size = T, d, layers, block_size
        self.store = SourceStore(T, d, s_max=MAX_SOURCES, dtype=torch.bfloat16, device=device)
        synth.fill_normal_(self.store.h0, h0_scale, seed=seed, tag=1)
        self.F = [synth.layer_output(T, d, std=layer_out_std, seed=seed, tag=l, device=device)
                  for l in range(layers)]
        self.W = [synth.query(d, seed=seed, device=device, tag=l) for l in range(layers)]
        # the queries are frozen parameters: prepared once for the two-phase pass
        self.W_split = block_queries_split(self.W, block_size)
        self.w_out = synth.query(d, seed=seed, device=device, tag=10_000)
        self.out = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.weights = torch.empty((T, MAX_SOURCES), dtype=torch.float32, device=device)
        self.final_out = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.final_weights = torch.empty((T, MAX_SOURCES), dtype=torch.float32, device=device)
        self._inter = None
        self._logits = None

    def step(self, on_layer=None, mode: str = "fused"):
        """One pass of the depth path.  ``mode``: ``"unfused"`` (aggregate +
        update per layer), ``"fused"`` (one launch per layer), ``"two_phase"``
        (blocks from ``TWO_PHASE_FROM`` on: one inter-block pass per block, one
        merge per later layer)."""
        self.store.reset()
        kw = {}
        if mode == "two_phase":
            if self._inter is None:
                dev = self.out.device
                self._inter = torch.empty((self.block_size, self.T, self.d), dtype=torch.bfloat16, device=dev)
                self._logits = torch.empty(self.block_size * self.T * 8, dtype=torch.float32, device=dev)
            kw = dict(two_phase_from=self.TWO_PHASE_FROM, inter=self._inter, logits=self._logits,
                      queries_split=self.W_split)
        elif mode not in ("fused", "unfused"):
            raise ValueError(f"unknown mode {mode!r}")
        run_schedule(self.store, self.F, self.W, self.block_size, out=self.out, weights=self.weights,
                     final_query=self.w_out, final_out=self.final_out, final_weights=self.final_weights,
                     on_layer=on_layer, fused=mode != "unfused", **kw)

    def capture(self, mode: str = "fused") -> "torch.cuda.CUDAGraph":
        """A HIP graph of one pass (``step(mode=mode)``): its launches recorded
        once and replayed with no host work -- for shapes where launching, not
        HBM, bounds a pass (decode).  A pass recomputes everything from h_0 and
        the layer outputs (each block's first layer copies its output into the
        partial slot), so every replay gives the same result as the eager pass.
        The library enqueues no memset, only kernels."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step(mode=mode)              # first use outside the capture
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step(mode=mode)
        return graph

    def source_counts(self):
        """S of every layer, then of the output layer."""
        counts, n_done, partial = [], 0, False
        for l in range(1, self.layers + 1):
            counts.append(1 + n_done + int(partial))
            partial = True
            if closes_block(l, self.layers, self.block_size):
                n_done, partial = n_done + 1, False
        return counts + [1 + n_done]

    def step_bytes(self, mode: str = "fused") -> int:
        """Algorithmic bytes of one full pass.  Unfused: every aggregation plus
        every update (copy for a block's first layer, read-modify-write
        otherwise).  Fused: each update's slot is not read back by the next
        aggregation, and a copy's source row is not read at all.  Two-phase
        blocks: one pass reading the n inter-block rows (and the closing
        update's rows) and writing B result rows + B*T*n logits, then per later
        layer the merge's rows (result row, layer output, old partial in;
        partial, residual out) and logits."""
        T, d = self.T, self.d
        row = 2 * T * d
        counts = self.source_counts()
        total = 0
        for l in range(1, self.layers + 1):
            n, i = (l - 1) // self.block_size + 1, (l - 1) % self.block_size + 1
            S = counts[l - 1]
            if mode == "two_phase" and n >= self.TWO_PHASE_FROM:
                if i == 1:
                    B = min(self.block_size, self.layers - l + 1)
                    prev_first = ((l - 2) % self.block_size == 0)   # closing a 1-layer partial: copy
                    total += (n - 1) * row                          # b's already complete + h_0
                    total += (1 if prev_first else 2) * row + row   # layer output (+ old partial) in, b_{n-1} out
                    total += B * row + B * T * n * 4 + B * d * 4 + T * n * 4
                else:
                    total += (2 if i >= 3 else 1) * row             # layer output (+ old partial) in
                    total += row + row + row                        # R in, partial out, residual out
                    total += T * n * 4 + T * (n + 1) * 4 + 4 * d
                continue
            total += T * (2 * S * d + 2 * d + 4 * S) + 4 * d
            if l > 1:
                first = (l - 2) % self.block_size == 0   # the update this launch fuses is a copy
                if mode == "unfused":
                    total += (2 if first else 3) * row
                else:
                    total += (1 if first else 2) * row
        # output layer (always fused with the last update, or an extra update)
        S = counts[-1]
        total += T * (2 * S * d + 2 * d + 4 * S) + 4 * d
        last_first = (self.layers - 1) % self.block_size == 0
        total += ((2 if last_first else 3) if mode == "unfused" else (1 if last_first else 2)) * row
        return total


class ManySources:
    """One aggregation over S > 9 sources (Full AttnRes: h_0 and every earlier
    layer output; S = 94 is K3's output layer) -- the batched online-softmax
    path.  Sources are N(0,1) * log-uniform scale like the other workloads."""

    def __init__(self, T: int, S: int = 94, d: int = 7168, *, seed: int = 0, device="cuda", scale=(0.5, 50.0)):
        self.T, self.S, self.d = T, S, d
        self.H = synth.sources(S, T, d, scale=scale, seed=seed, device=device)
        self.w = synth.query(d, seed=seed, device=device)
        self.out = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.weights = torch.empty((T, S), dtype=torch.float32, device=device)

    def step(self):
        from .binding import aggregate
        aggregate(self.H, self.w, self.out, self.weights)

    def step_bytes(self) -> int:
        S, T, d = self.S, self.T, self.d
        return T * (2 * S * d + 2 * d + 4 * S) + 4 * d


class LayerBackward:
    """One aggregation's backward at S = 9 (h_0, seven block representations,
    the partial sum): recompute the forward, add every source's gradient into
    its float32 gradient row, hand out the last source's new gradient (bf16),
    and reduce dL/dw over the tokens -- one ``attnres_aggregate_backward``."""

    def __init__(self, T: int, d: int = 7168, *, seed: int = 0, device="cuda", scale=(0.5, 50.0)):
        from .binding import backward_workspace_bytes
        self.T, self.d, self.S = T, d, MAX_SOURCES
        self.H = synth.sources(self.S, T, d, scale=scale, seed=seed, device=device)
        self.w = synth.query(d, seed=seed, device=device)
        self.g = synth.layer_output(T, d, std=1.0, seed=seed, tag=3, device=device)
        self.grads = torch.zeros((self.S, T, d), dtype=torch.float32, device=device)
        self.grad_last = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.grad_w = torch.empty(d, dtype=torch.float32, device=device)
        nbytes = backward_workspace_bytes(T, d)
        self.workspace = torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device=device)

    def step(self):
        from .binding import aggregate_backward
        aggregate_backward(self.H, self.w, self.g, self.grads, accumulate=(1 << self.S) - 1, grad_w=self.grad_w,
                           grad_last=self.grad_last, workspace=self.workspace)

    def step_bytes(self) -> int:
        """Sources and g in, float32 gradient rows read and written, the last
        source's gradient out (bf16), the query in and dL/dw out."""
        S, T, d = self.S, self.T, self.d
        return T * (2 * S * d + 2 * d + 8 * S * d + 2 * d) + 8 * d


class ScheduleBackward:
    """The backward of the whole 93-layer schedule at one batch of tokens: the
    output layer's aggregation, then layers 93..1 in reverse, each block's
    partial sums recomputed, every source gradient accumulated in float32 and
    each layer output's finished gradient handed out (bf16).  The forward
    (outside the timed region) leaves h_0 and the block representations in the
    store; dL/dr_l are synthetic inputs."""

    def __init__(self, T: int, d: int = 7168, *, layers: int = 93, block_size: int = 12, seed: int = 0,
                 device="cuda"):
        self.fwd = Schedule(T, d, layers=layers, block_size=block_size, seed=seed, device=device)
        self.T, self.d, self.layers, self.block_size = T, d, layers, block_size
        self.fwd.step(mode="fused")
        self.dr = [synth.layer_output(T, d, std=1.0, seed=seed, tag=5000 + l, device=device) for l in range(layers)]
        self.dr_final = synth.layer_output(T, d, std=1.0, seed=seed, tag=6000, device=device)
        nblocks = (layers + block_size - 1) // block_size
        self.grad_store = torch.empty((1 + nblocks, T, d), dtype=torch.float32, device=device)
        self.grad_w = [torch.empty(d, dtype=torch.float32, device=device) for _ in range(layers)]
        self.grad_w_final = torch.empty(d, dtype=torch.float32, device=device)

    def step(self, on_grad=None):
        from .schedule import run_schedule_backward
        run_schedule_backward(self.fwd.store, self.fwd.F, self.fwd.W, self.block_size, self.dr,
                              final_query=self.fwd.w_out, grad_final=self.dr_final, grad_store=self.grad_store,
                              grad_w=self.grad_w, grad_w_final=self.grad_w_final, on_grad=on_grad)

    def step_bytes(self, defer: bool = True) -> int:
        """Algorithmic bytes of one backward pass.  Every layer reads its
        sources and dL/dr and hands out a gradient; with ``defer`` a layer
        updates only its partial's gradient row and writes 3 coefficients per
        token and source (its dL/dw is formed per block), and one pass per
        block reads the block's inter-block sources, its dL/dr rows and
        coefficients and writes each inter-block gradient row once
        (read-modify-write, except in the last block, whose rows the deferred
        output layer leaves untouched); the output layer is one more layer of
        the last block's pass.  Without ``defer`` every layer
        read-modify-writes all its sources' gradient rows and writes its dL/dw.
        Not counted: the second reads of rows by the dL/dw contractions (an
        implementation choice: a block's n inter-block sources and the B - 1
        partial sums, once more per block)."""
        T, d, L, bs = self.T, self.d, self.layers, self.block_size
        row2, row4 = 2 * T * d, 4 * T * d
        nblocks = (L + bs - 1) // bs
        # output layer: sources and g in, dF out; gradient rows written first touch
        # (only b_N's when the other sources are deferred to the last block's pass)
        S = 1 + nblocks
        total = S * row2 + row2 + row2 + 4 * d          # sources, g, dF out; query in
        total += (row4 + 12 * S * T) if defer else (S * row4 + 4 * d)   # (+ dL/dw out when formed here)
        for n in range(1, nblocks + 1):
            B = min(n * bs, L) - (n - 1) * bs
            if B >= 2:                                   # partial sums recomputed in one pass
                total += 2 * (B - 1) * row2
            for i in range(1, B + 1):
                S = n + (1 if i >= 2 else 0)
                total += S * row2 + row2 + 4 * d             # sources, g; query in
                if defer:
                    total += 12 * S * T                      # coefficients of every source
                    if i >= 2:
                        total += 2 * row4 + row2             # the partial's gradient row, dF out
                else:
                    total += 2 * S * row4 + row2 + 4 * d     # every gradient row, dF out, dL/dw out
            if defer:                                        # one pass per block (+ the output layer in the last)
                Bc = B + (1 if n == nblocks else 0)
                rows = n * row4 if n == nblocks else 2 * n * row4
                total += n * row2 + Bc * row2 + 12 * n * Bc * T + rows + row2 + 12 * d * Bc
                # the partial sums' share of dL/dw: each layer's own last source's
                # c1 in, every layer's dL/dw row written (its row re-read: not counted)
                total += 4 * T * (Bc - 1) + 4 * d * Bc
        return total
