"""Per-layer depth schedule of a Block AttnRes stack (host bookkeeping only).

kimi.papertok.ai ch. 4 §4.3 (eq 10) and §4.5: layers are grouped into blocks of
``block_size``; layer i of block n aggregates over h_0, b_1..b_{n-1} and, from
i = 2 on, the block's partial sum; after the layer its output is added to the
partial, and the block's last layer closes it (§4.6: the representation is
produced once at the boundary and then stays resident).  The output layer
aggregates h_0 and every block representation (§4.3, last paragraph).

``run_schedule`` drives the forward through the C ABI -- per layer (an
aggregation and a partial-sum update, or both fused in one launch) or, from a
chosen block on, two-phase (one pass over a block's inter-block sources for
all its queries, then one merge per layer); ``run_full_schedule`` drives Full
AttnRes; ``run_schedule_backward`` the backward in reverse layer order.  The
only host work is bookkeeping: which sources a layer sees, the finalize flags
and the buffers.
"""

from __future__ import annotations

from typing import Callable, Optional, Sequence

import torch

from . import markers
from .binding import MAX_BLOCK_QUERIES, MAX_INTER_SOURCES, SourceStore, aggregate, split_queries


def closes_block(layer: int, num_layers: int, block_size: int) -> bool:
    """True if 1-based ``layer`` is the last layer of its block."""
    return layer % block_size == 0 or layer == num_layers


def block_queries_split(queries: Sequence[torch.Tensor], block_size: int):
    """:func:`split_queries` of every block's queries (list indexed by block - 1)."""
    L = len(queries)
    return [split_queries(torch.stack(list(queries[l0:min(l0 + block_size, L)])))
            for l0 in range(0, L, block_size)]


def run_schedule(store: SourceStore, layer_outputs: Sequence[torch.Tensor], queries: Sequence[torch.Tensor],
                 block_size: int, *, out: Optional[torch.Tensor] = None, weights: Optional[torch.Tensor] = None,
                 final_query: Optional[torch.Tensor] = None, final_out: Optional[torch.Tensor] = None,
                 final_weights: Optional[torch.Tensor] = None,
                 on_layer: Optional[Callable[[int, torch.Tensor, Optional[torch.Tensor]], None]] = None,
                 fused: bool = True, two_phase_from: Optional[int] = None,
                 inter: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                 queries_split: Optional[Sequence[Optional[torch.Tensor]]] = None, eps: float = 1e-5):
    """Run every layer's aggregation and partial-sum update in stream order.

    Per layer one of:
      * ``fused=False``: ``attnres_aggregate`` then ``attnres_accumulate`` (2L+1
        launches);
      * default: layer 1 aggregates h_0 alone; every later layer l is one
        ``attnres_accumulate_aggregate`` that adds F_{l-1} (closing its block
        when it was the block's last layer) and aggregates with w_l;
      * ``two_phase_from=n0``: blocks n >= n0 run the two-phase schedule --
        one ``attnres_block_prepare`` (closing the previous block, then one pass
        over h_0, b_1..b_{n-1} for all the block's queries -- one pass per 16
        queries for longer blocks; its first query's result is the block's first
        residual) and one ``attnres_block_merge``
        per later layer; other blocks run as in the default.
    The output layer's aggregation is fused with the last update.  All modes
    agree with the oracle; the fused and unfused ones bit for bit with each
    other.

    ``store`` must hold h_0 in slot 0 and no blocks yet.  ``out`` is either one
    ``[T, d]`` buffer reused by every layer or ``[L, T, d]``; ``weights``
    likewise ``[T, 9]`` (each layer writes a ``[T, S_l]`` block at its start) or
    ``[L, T, 9]``.  Two-phase blocks need ``inter`` ``[block_size, T, d]`` (store
    dtype) and ``logits`` (float32, ``block_size * T * 8`` elements) unless
    ``out`` is ``[L, T, d]``, whose rows then hold the pass's results directly;
    ``queries_split[n-1]`` (:func:`split_queries` of block n's queries, done
    once since the queries are frozen parameters) saves the split per pass;
    ``block_queries_split`` builds that list.
    ``on_layer(l, r_l, a_l)`` runs after layer l's aggregation is enqueued
    (1-based l).  Returns the output layer's ``(out, weights)`` when
    ``final_query`` is given, else None.
    """
    num_layers = len(layer_outputs)
    if len(queries) != num_layers or num_layers == 0:
        raise ValueError("one query per layer, at least one layer")
    if store.n_completed != 0 or store.partial_valid:
        raise ValueError("store must start with only h_0 live")
    T, d = store.T, store.d
    dev = store.slots.device
    if out is None:
        out = torch.empty((T, d), dtype=store.slots.dtype, device=dev)

    def wview(l: int, S: int):
        if weights is None:
            return None
        wbuf = weights[l - 1] if weights.dim() == 3 else weights
        return wbuf.view(-1)[: T * S].view(T, S)

    def rbuf(l: int):
        return out[l - 1] if out.dim() == 3 else out

    if not fused:
        for l in range(1, num_layers + 1):
            with markers.span("layer", l):
                r, a = rbuf(l), wview(l, store.num_sources())
                aggregate(store.sources(), queries[l - 1], r, a, want_weights=a is not None, eps=eps)
            if on_layer is not None:
                on_layer(l, r, a)
            with markers.span("update", l):
                store.accumulate(layer_outputs[l - 1], closes_block(l, num_layers, block_size))
        if final_query is not None:
            with markers.span("output layer"):
                return aggregate(store.sources(), final_query, final_out, final_weights, eps=eps)
        return None

    num_blocks = (num_layers + block_size - 1) // block_size
    two_phase = set()
    if two_phase_from is not None:
        two_phase = {n for n in range(max(1, two_phase_from), num_blocks + 1) if n <= MAX_INTER_SOURCES}
        if two_phase and out.dim() != 3 and (inter is None or logits is None):
            inter = torch.empty((block_size, T, d), dtype=store.slots.dtype, device=dev)
            logits = torch.empty(block_size * T * MAX_INTER_SOURCES, dtype=torch.float32, device=dev)

    block_rows = None   # R rows of the current two-phase block
    block_logits = None
    for l in range(1, num_layers + 1):
        n, i = (l - 1) // block_size + 1, (l - 1) % block_size + 1
        last = min(n * block_size, num_layers)
        with markers.span("layer", l):
            if n in two_phase and i == 1:
                B = last - l + 1
                K = n  # h_0 and b_1..b_{n-1} once the previous block is closed
                if queries_split is not None and queries_split[n - 1] is not None:
                    W = queries_split[n - 1]
                else:
                    W = split_queries(torch.stack([queries[j] for j in range(l - 1, last)]))
                block_rows = out[l - 1:last] if out.dim() == 3 else inter[:B]
                lg_buf = logits if out.dim() != 3 else None
                if lg_buf is None:
                    lg_buf = torch.empty(B * T * K, dtype=torch.float32, device=dev)
                block_logits = lg_buf[: B * T * K].view(B, T, K)
                a = wview(l, K)
                # one pass per MAX_BLOCK_QUERIES queries (groups of four in W); only
                # the first closes the previous block
                for q0 in range(0, B, MAX_BLOCK_QUERIES):
                    q1 = min(q0 + MAX_BLOCK_QUERIES, B)
                    first = q0 == 0
                    with markers.span("inter-block pass of block", n):
                        store.block_prepare(layer_outputs[l - 2] if first and l > 1 else None, first and l > 1,
                                            W[q0 // 4:(q1 + 3) // 4], block_rows[q0:q1], block_logits[q0:q1],
                                            a if first else None, eps=eps)
                r = block_rows[0]
            elif n in two_phase:
                a = wview(l, n + 1)
                r = rbuf(l)
                store.block_merge(layer_outputs[l - 2], queries[l - 1], block_rows[i - 1], block_logits[i - 1],
                                  out=r, weights=a, want_weights=a is not None, eps=eps)
            elif l == 1:
                r, a = rbuf(l), wview(l, store.num_sources())
                aggregate(store.sources(), queries[0], r, a, want_weights=a is not None, eps=eps)
            else:
                closes = closes_block(l - 1, num_layers, block_size)
                S = 1 + store.n_completed + (1 if closes else 0) + (0 if closes else 1)
                r, a = rbuf(l), wview(l, S)
                store.accumulate_aggregate(layer_outputs[l - 2], closes, queries[l - 1], r, a,
                                           want_weights=a is not None, eps=eps)
        if on_layer is not None:
            on_layer(l, r, a)
    with markers.span("output layer"):
        if final_query is not None:
            return store.accumulate_aggregate(layer_outputs[-1], True, final_query, final_out, final_weights, eps=eps)
        store.accumulate(layer_outputs[-1], True)
    return None


def run_full_schedule(sources: torch.Tensor, queries: Sequence[torch.Tensor], *, out: Optional[torch.Tensor] = None,
                      weights: Optional[torch.Tensor] = None, final_query: Optional[torch.Tensor] = None,
                      final_out: Optional[torch.Tensor] = None, final_weights: Optional[torch.Tensor] = None,
                      on_layer: Optional[Callable[[int, torch.Tensor, Optional[torch.Tensor]], None]] = None,
                      eps: float = 1e-5):
    """Full AttnRes (kimi.papertok.ai ch. 4 §4.2): layer l aggregates h_0 and the
    outputs of every earlier layer.  ``sources`` is ``[L + 1, T, d]`` with h_0 in
    row 0 and layer l's output in row l (a layer writes its output straight
    into its row, so nothing is copied); layer l reads rows ``[0, l)`` -- one
    ``attnres_aggregate`` with S = l, batched online softmax beyond 9 rows.
    ``out``/``weights`` as in :func:`run_schedule` (``weights`` rows hold up to
    L + 1 columns).  Returns the output layer's ``(out, weights)`` over all
    L + 1 rows when ``final_query`` is given."""
    num_layers = len(queries)
    if sources.dim() != 3 or sources.shape[0] < num_layers + (1 if final_query is not None else 0):
        raise ValueError("sources must be [L + 1, T, d]")
    T, d = sources.shape[1], sources.shape[2]
    if out is None:
        out = torch.empty((T, d), dtype=sources.dtype, device=sources.device)
    for l in range(1, num_layers + 1):
        r = out[l - 1] if out.dim() == 3 else out
        a = None
        if weights is not None:
            wbuf = weights[l - 1] if weights.dim() == 3 else weights
            a = wbuf.view(-1)[: T * l].view(T, l)
        aggregate(sources[:l], queries[l - 1], r, a, want_weights=a is not None, eps=eps)
        if on_layer is not None:
            on_layer(l, r, a)
    if final_query is not None:
        return aggregate(sources[: num_layers + 1], final_query, final_out, final_weights, eps=eps)
    return None


def run_schedule_backward(store: SourceStore, layer_outputs: Sequence[torch.Tensor], queries: Sequence[torch.Tensor],
                          block_size: int, grad_r, *, final_query: Optional[torch.Tensor] = None,
                          grad_final: Optional[torch.Tensor] = None, grad_store: Optional[torch.Tensor] = None,
                          grad_w: Optional[Sequence[torch.Tensor]] = None, grad_w_final: Optional[torch.Tensor] = None,
                          on_grad: Optional[Callable[[int, torch.Tensor], None]] = None, defer: bool = True,
                          eps: float = 1e-5):
    """Backward of ``run_schedule``, layer by layer in reverse, recomputing each
    block's partial sums (kimi.papertok.ai §4.6: the aggregation is
    recomputed in the backward pass).

    ``store`` is the forward's store after the pass (h_0 and every block
    representation; left unchanged).  Each block's partial sums are recomputed
    into a buffer of their own and passed to the layer's backward as its last
    source (one ``attnres_partial_sums`` pass per block).  ``grad_r`` is a sequence of dL/dr_l ``[T, d]`` (store dtype) or a
    callable ``grad_r(l, dF_l) -> dL/dr_l``: the layer's own backward, given
    the finished gradient of its output.  Gradients of the sources accumulate in
    ``grad_store`` ``[1 + blocks, T, d]`` float32: row 0 is dL/dh_0, row n the
    gradient of block n's representation, which is also the running gradient
    of its partial sums.  ``on_grad(l, dF_l)`` receives each layer output's
    finished gradient (store dtype), l = L..0 where dF_0 is dL/dh_0 rounded.

    With ``defer`` (default) the gradients of a block's inter-block sources
    (h_0, b_1 .. b_{n-1}, shared by all its layers) are not updated per layer:
    each layer's backward writes three coefficients per token and source, and
    one ``attnres_block_backward`` per block applies them -- one
    read-modify-write of those rows per block instead of one per layer -- and
    adds those sources' share of each layer's dL/dw.  The layers' backwards
    form no dL/dw themselves (one workgroup per token, nothing summed over
    tokens): they also write the coefficients of their partial sum, whose
    share of each layer's dL/dw one ``attnres_partial_dw`` per block forms
    from the block's recomputed partial sums.  The final aggregation's sources
    h_0 .. b_{N-1} are the last block's inter-block sources, so it joins that
    block's pass as one more layer.
    Returns ``(grad_store, grad_w, grad_w_final)``.
    """
    from .binding import aggregate_backward, block_backward, partial_dw, partial_sums

    L = len(layer_outputs)
    T, d = store.T, store.d
    dev, dt = store.slots.device, store.slots.dtype
    nblocks = (L + block_size - 1) // block_size
    if store.n_completed != nblocks or store.partial_valid:
        raise ValueError("store must hold h_0 and every block representation (the forward's end state)")
    if grad_store is None:
        grad_store = torch.empty((1 + nblocks, T, d), dtype=torch.float32, device=dev)
    if grad_w is None:
        grad_w = [torch.empty(d, dtype=torch.float32, device=dev) for _ in range(L)]
    if final_query is not None and grad_w_final is None:
        grad_w_final = torch.empty(d, dtype=torch.float32, device=dev)
    slots = store.slots
    dF = torch.empty((T, d), dtype=dt, device=dev)
    partials = torch.empty((block_size, T, d), dtype=dt, device=dev)  # partials[i-2]: before position i
    # per token of block n: Bc layer slots of n + 1 triples (the n inter-block
    # sources, then the layer's own last source)
    coef_all = (torch.empty(T * (block_size + 1) * (nblocks + 1) * 3, dtype=torch.float32, device=dev)
                if defer else None)
    holds = [False] * (1 + nblocks)   # which gradient rows already hold a gradient
    final_in_block = defer and final_query is not None

    def acc_mask(rows):
        return sum(1 << k for k, r in enumerate(rows) if holds[r])

    def dr(l):
        return grad_r(l, dF) if callable(grad_r) else grad_r[l - 1]

    def block_layers(n):
        return min(n * block_size, L) - (n - 1) * block_size + (1 if final_in_block and n == nblocks else 0)

    def block_coef(n):
        Bc = block_layers(n)
        return coef_all[:T * Bc * (n + 1) * 3].view(T, Bc, n + 1, 3)

    with markers.span("output layer backward"):
        if final_query is not None:
            S = 1 + nblocks
            if final_in_block:
                # h_0 .. b_{N-1} deferred to the last block's pass (its last layer
                # slot); only b_N's gradient row is written here
                N, Bc = nblocks, block_layers(nblocks)
                m = 3 * (N + 1)
                aggregate_backward(slots[:S], final_query, grad_final, grad_store[:S], accumulate=0,
                                   defer=(1 << N) - 1, coef=block_coef(N).view(-1)[m * (Bc - 1):],
                                   coef_stride=m * Bc, form_dw=False, grad_last=dF, eps=eps)
                holds[N] = True
            else:
                aggregate_backward(slots[:S], final_query, grad_final, grad_store[:S], accumulate=acc_mask(range(S)),
                                   grad_w=grad_w_final, grad_last=dF, eps=eps)
                holds[:S] = [True] * S
        else:
            dF.zero_()
    if on_grad is not None:
        on_grad(L, dF)
    for n in range(nblocks, 0, -1):
        first = (n - 1) * block_size + 1
        last = min(n * block_size, L)
        B = last - first + 1
        # the block's partial sums, formed exactly as the forward formed them
        if B >= 2:
            with markers.span("partial sums of block", n):
                partial_sums([layer_outputs[j - 1] for j in range(first, last)], partials)
        coef = block_coef(n) if defer else None
        Bc = coef.shape[1] if defer else B
        m = 3 * (n + 1)    # coefficient floats per layer slot and token
        block_g = [None] * B
        for l in range(last, first - 1, -1):
            i = l - first + 1
            g = dr(l)
            block_g[i - 1] = g
            # deferred: coefficients of every source out, dL/dw formed per block
            cf = (dict(defer=(1 << n) - 1, coef=coef.view(-1)[m * (i - 1):], coef_stride=m * Bc, form_dw=False)
                  if defer else dict(grad_w=grad_w[l - 1]))
            with markers.span("layer backward", l):
                if i >= 2:
                    rows = list(range(n + 1))
                    aggregate_backward(slots[:n], queries[l - 1], g, grad_store[:n + 1], last_source=partials[i - 2],
                                       accumulate=acc_mask(rows), grad_last=dF, eps=eps, **cf)
                    touched = rows if not defer else [n]
                else:
                    rows = list(range(n))
                    aggregate_backward(slots[:n], queries[l - 1], g, grad_store[:n], accumulate=acc_mask(rows),
                                       grad_last=None if defer else dF, eps=eps, **cf)
                    touched = [] if defer else rows
            for r in touched:
                holds[r] = True
            if on_grad is not None and (i >= 2 or not defer):
                on_grad(l - 1, dF)
        if defer:
            qs = [queries[j - 1] for j in range(first, last + 1)]
            dws = [grad_w[j - 1] for j in range(first, last + 1)]
            # each layer's own last source: its partial sum (none for the block's first layer)
            own = [None] + [partials[i - 2] for i in range(2, B + 1)]
            if Bc > B:   # the final aggregation, in the last slot; its own last source is b_N
                block_g, qs, dws = block_g + [grad_final], qs + [final_query], dws + [grad_w_final]
                own = own + [slots[n]]
            with markers.span("gradient rows of block", n):
                # the partials' share of dL/dw (written), then the inter-block sources' (added)
                partial_dw(own, coef.view(-1)[3 * n + 1:], m * Bc, m, dws)
                block_backward(slots[:n], block_g, qs, coef, grad_store[:n], dws, accumulate=acc_mask(range(n)),
                               grad_last=dF, coef_layer_stride=m)
            holds[:n] = [True] * n
            if on_grad is not None:
                on_grad(first - 1, dF)
    return grad_store, grad_w, grad_w_final
