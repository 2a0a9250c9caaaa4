"""Plain CPU oracle for the Block Attention-Residuals (Block AttnRes) depth aggregation.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only the tests, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and imports nothing from
it.  Everything here is float64 NumPy, written for a reader to check against the
pages by eye, not for speed: no blocking, fusion, online softmax or reordering.

Pages cited below (titles as published; section, equation or figure named):

* [TUT]   "Kimi K3" technical-report tutorial, kimi.papertok.ai -- ch. 0 §0.7
          (softmax), §0.11 (RMSNorm); ch. 4 "Attention Residuals" §4.2 (eq 8-9),
          §4.3 (eq 10), §4.4, §4.5, §4.6.
* [BLOG2] "Kimi K3技术详解系列（二）：AttnRes 与 Stable LatentMoE" -- §2 (the
          depth-attention definition and its three-line listing), §2.1 (the
          four-layer worked example), §3 (Block AttnRes and its diagram).
* [BLOG6] "Kimi K3 模型结构（6）：输入端与零件" -- the list of loose model facts
          (RMSNorm eps is 1e-5 throughout the model).
* [ATLAS] llm-atlas.k1412.top/k3 -- card "07 ATTENTION RESIDUALS" (the
          alpha_{i->l} formula; 8 layer blocks + embedding = 9 sources), the
          "save per block" source-count widget, and the study of the parameter-free
          uniform mixer (zero logits give weight 1/N).

Readings where the pages are silent or garbled (each also listed in the design
notes): eps sits inside the square root; the RMSNorm has no gain; there is no
temperature; values are the raw sources; the first layer of a block has no
partial source at all; a block representation is the plain sum of its layers'
outputs; a bf16 store forms each partial sum in float32 and rounds it to bf16
with round-to-nearest-even.  Backward: the pages give no formula, only that
training recomputes the aggregation ([TUT] §4.6) and that the gradient
reaches a source along a value path and a softmax/query/key path ([ATLAS]
study of the spike trajectory x backward path); the gradient here is the exact
derivative of the forward definition, and the rounding of a stored sum passes
gradients through unchanged.

Parity pins (tests that fix this oracle to something other than itself):
every function below is pinned -- the worked example of [BLOG2] §2.1, a
library reduction (torch ``rms_norm`` + ``scaled_dot_product_attention``, up to
94 sources), closed forms (S=1, zero query, equal sources, S=2 logistic),
invariants, 50-digit brute force, bf16 rounding against torch and hand-made
ties, the schedule's source counts from [TUT] §4.5 / [ATLAS]'s widget, and
([TUT] §4.3) Block AttnRes with one layer per block being Full AttnRes.
Backward: torch autograd through the library reduction, central finite
differences, closed forms (one source, zero query, identical sources), the
rescaling invariant, and autograd through a whole Block AttnRes schedule with
exact partial sums.  None is marked "parity unpinned".
"""

from __future__ import annotations

import numpy as np

#: RMSNorm epsilon, the same everywhere in the model ([BLOG6], loose facts).
EPS = 1e-5


# ----------------------------------------------------------------------------
# Definition of one depth aggregation ([BLOG2] §2; [TUT] §4.2 eq 8-9;
# [ATLAS] card 07).
# ----------------------------------------------------------------------------

def rmsnorm(x, eps: float = EPS) -> np.ndarray:
    """Gain-free RMSNorm over the last axis, in float64.

    [TUT] §0.11: square every entry, average, take the square root, divide each
    entry by it.  eps ([BLOG6]) is added to the mean square inside the root.
    No learned gain: the pages show none, and a per-channel gain would fold
    into the pseudo-query anyway.
    """
    x = np.asarray(x, dtype=np.float64)
    mean_square = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(mean_square + eps)


def softmax(z, axis: int = -1) -> np.ndarray:
    """[TUT] §0.7: exponentiate each score, divide by the sum of the exponentials.

    The maximum is subtracted before exponentiating; this leaves the result
    unchanged and keeps large scores finite.
    """
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=axis, keepdims=True))
    return e / np.sum(e, axis=axis, keepdims=True)


def depth_attention(H, w, eps: float = EPS):
    """One AttnRes aggregation per token, as [BLOG2] §2 defines it.

    keys = RMSNorm(H);  a = softmax over sources of (w . key);  r = sum_s a_s H_s.

    The pseudo-query ``w`` belongs to the layer, not to the token ([TUT] §4.2);
    keys and values are the same source vectors, normalised only inside the
    score ([TUT] §4.2: phi(q, k) = exp(q^T RMSNorm(k)), no temperature).

    Args:
      H: ``[S, T, d]`` sources, source-major (h_0, block representations,
         partial sum), any real dtype; upcast exactly to float64.
      w: ``[d]`` pseudo-query.
    Returns:
      ``(r, a)``: residual ``[T, d]`` and depth weights ``[T, S]``, float64.
    """
    H = np.asarray(H, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if H.ndim != 3 or w.shape != (H.shape[2],):
        raise ValueError("H must be [S, T, d] and w must be [d]")
    keys = rmsnorm(H, eps)                 # [S, T, d]
    logits = (keys @ w).T                  # [T, S]: w . RMSNorm(H_s) per token
    a = softmax(logits, axis=1)            # softmax over depth
    r = np.zeros(H.shape[1:], dtype=np.float64)
    for s in range(H.shape[0]):            # weighted sum of the RAW sources
        r += a[:, s:s + 1] * H[s]
    return r, a


# ----------------------------------------------------------------------------
# bfloat16 storage: bf16 is the top half of an IEEE binary32 word.
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns, round-to-nearest-even.

    The low 16 bits are dropped after adding half of the dropped range, plus one
    more when the kept part is odd (ties go to the even pattern).  NaNs stay
    NaN (quiet bit set); overflow rounds to infinity.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    kept_lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + kept_lsb) >> 16
    bits = np.where(is_nan, (u >> 16) | 0x0040, rounded) & 0xFFFF
    return bits.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_round(x) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------
# Block AttnRes bookkeeping ([TUT] §4.3 eq 10, §4.5, §4.6; [BLOG2] §3).
# ----------------------------------------------------------------------------

def accumulate(partial, layer_out, dtype: str):
    """Add one layer's output into its block's partial sum.

    [TUT] §4.3: inside a block the layers' outputs are summed into one block
    representation; the partial sum runs up to the previous layer ([BLOG2] §3).
    ``partial=None`` means the block has no partial yet (its first layer): the
    result is the layer output itself.

    ``dtype='bf16'``: inputs are float32 arrays holding bf16 values; the sum is
    one float32 addition (IEEE, ties to even), then rounded to bf16 -- the
    precision of a bf16 store.  ``dtype='f32'``: one float32 addition.
    """
    layer_out = np.asarray(layer_out, dtype=np.float32)
    if partial is None:
        return layer_out.copy()
    total = np.asarray(partial, dtype=np.float32) + layer_out   # float32 add
    if dtype == "bf16":
        return bf16_round(total)
    if dtype == "f32":
        return total
    raise ValueError(f"unknown dtype {dtype!r}")


def block_layout(num_layers: int, block_size: int):
    """(block n, position i) of every layer l = 1..num_layers, both 1-based.

    [TUT] §4.3: the L layers are cut into blocks of consecutive layers; §4.5:
    K3's 93 layers in blocks of 12 give 8 blocks, the last one incomplete.
    """
    return [((l - 1) // block_size + 1, (l - 1) % block_size + 1)
            for l in range(1, num_layers + 1)]


def layer_source_names(block: int, position: int):
    """Sources layer i of block n attends over ([TUT] §4.3 eq 10; [BLOG2] §3).

    Always h_0 and the completed block representations b_1..b_{n-1}; from the
    block's second layer on, also the partial sum of the block's earlier
    layers.  The first layer gets no partial entry at all -- not a zero vector,
    which would still take a slot and a share of the weight ([TUT] §4.3).
    """
    names = ["h0"] + [f"b{k}" for k in range(1, block)]
    if position >= 2:
        names.append("partial")
    return names


def run_schedule(h0, layer_outputs, queries, block_size: int, dtype: str,
                 final_query=None, eps: float = EPS):
    """Forward the depth path of a Block AttnRes stack, layer by layer.

    For l = 1..L: aggregate over the sources of ``layer_source_names`` with
    query ``queries[l-1]`` (giving r_l), then add ``layer_outputs[l-1]`` into the
    block's partial sum; the partial becomes the block representation b_n once
    the block's last layer has been added ([TUT] §4.6: produced once at the
    block boundary and shared by all later layers).  If ``final_query`` is
    given, the output layer aggregates h_0 and all block representations
    ([TUT] §4.3, last paragraph).

    Layer outputs are inputs here (synthetic), not functions of r_l.

    Args:
      h0: ``[T, d]`` embedding source.  layer_outputs: ``[L, T, d]``.
      queries: ``[L, d]``.  dtype: store precision, ``'bf16'`` or ``'f32'``.
    Returns:
      dict with ``r`` (list of ``[T, d]`` float64), ``a`` (list of ``[T, S_l]``),
      ``num_sources`` (list of S_l), ``blocks`` (list of ``[T, d]`` float32
      block representations in store precision) and, with ``final_query``,
      ``final_r`` / ``final_a``.
    """
    h0 = np.asarray(h0, dtype=np.float32)
    num_layers = len(layer_outputs)
    blocks, partial = [], None
    out = {"r": [], "a": [], "num_sources": []}
    for (n, i), F, w in zip(block_layout(num_layers, block_size), layer_outputs, queries):
        if i == 1:
            partial = None
        named = {"h0": h0, "partial": partial}
        named.update({f"b{k + 1}": b for k, b in enumerate(blocks)})
        H = np.stack([named[name] for name in layer_source_names(n, i)])
        r, a = depth_attention(H, w, eps)
        out["r"].append(r)
        out["a"].append(a)
        out["num_sources"].append(H.shape[0])
        partial = accumulate(partial, F, dtype)
        block_ends = (i == block_size) or (len(out["r"]) == num_layers)
        if block_ends:
            blocks.append(partial)
            partial = None
    out["blocks"] = blocks
    if final_query is not None:
        H = np.stack([h0] + blocks)
        out["final_r"], out["final_a"] = depth_attention(H, final_query, eps)
    return out


def run_full_schedule(h0, layer_outputs, queries, final_query=None, eps: float = EPS):
    """Full AttnRes ([TUT] §4.2): layer l aggregates h_0 and the outputs of every
    earlier layer, h_1..h_{l-1}, with its own query; the output layer (if
    ``final_query`` is given) aggregates all L + 1.  Sources are kept at their
    given precision.  Returns the list of ``(r_l, a_l)`` and, optionally, the
    output layer's pair."""
    sources = [np.asarray(h0, dtype=np.float32)]
    per_layer = []
    for F, w in zip(layer_outputs, queries):
        per_layer.append(depth_attention(np.stack(sources), w, eps))
        sources.append(np.asarray(F, dtype=np.float32))
    final = depth_attention(np.stack(sources), final_query, eps) if final_query is not None else None
    return per_layer, final


# ----------------------------------------------------------------------------
# Backward: the derivative of depth_attention, then of the Block AttnRes
# schedule.  The pages fix no formula; training recomputes the aggregation
# ([TUT] §4.6), and the gradient reaches each source along a value path (the
# weight times the upstream gradient) and along the softmax / query / key path
# ([ATLAS] study of the spike trajectory x backward path).  Written as the chain
# rule through the forward's steps, in the forward's order.
# ----------------------------------------------------------------------------

def depth_attention_backward(H, w, g, eps: float = EPS, per_source: bool = False):
    """Gradients of ``L = sum_t g[t] . r[t]`` for ``r, a = depth_attention(H, w)``.

    Args:
      H: ``[S, T, d]`` sources; w: ``[d]`` query; g: ``[T, d]`` upstream
         gradient dL/dr.  Any real dtype, upcast to float64.
      per_source: also return each source's share of dL/dw -- the gradient
         reaching w through that source's logit alone, ``sum_t dz_s k_s``.
    Returns:
      ``(dH, dw)``: ``[S, T, d]`` and ``[d]`` (summed over tokens), float64;
      with ``per_source``, ``(dH, dw, dw_src)`` with ``dw_src`` ``[S, d]``.
    """
    H = np.asarray(H, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    S, T, d = H.shape
    # forward, recomputed step by step
    mean_square = np.mean(H * H, axis=-1, keepdims=True)           # [S, T, 1]
    rms = np.sqrt(mean_square + eps)
    keys = H / rms                                                  # [S, T, d]
    logits = (keys @ w).T                                           # [T, S]
    a = softmax(logits, axis=1)                                     # [T, S]
    # r = sum_s a_s H_s: value path, and the gradient of each weight
    dH = np.zeros_like(H)
    da = np.zeros((T, S))
    for s in range(S):
        dH[s] += a[:, s:s + 1] * g                                  # value path
        da[:, s] = np.sum(g * H[s], axis=1)                         # dL/da_s = g . H_s
    # softmax over sources: dz_s = a_s (da_s - sum_s' a_s' da_s')
    dz = a * (da - np.sum(a * da, axis=1, keepdims=True))          # [T, S]
    # logits = keys . w
    dw = np.zeros(d)
    dw_src = np.zeros((S, d))
    dkeys = np.zeros_like(H)
    for s in range(S):
        dw_src[s] = np.sum(dz[:, s:s + 1] * keys[s], axis=0)
        dw += dw_src[s]
        dkeys[s] = dz[:, s:s + 1] * w
    # keys = H / sqrt(mean(H^2) + eps): dH = (dkeys - keys * mean(dkeys * keys)) / rms
    dH += (dkeys - keys * np.mean(dkeys * keys, axis=-1, keepdims=True)) / rms
    return (dH, dw, dw_src) if per_source else (dH, dw)


def layer_sources(h0, layer_outputs, block_size: int, dtype: str):
    """Per layer: the names and stacked sources it aggregates (as the store holds
    them, partial sums rounded to ``dtype``), plus the block representations."""
    h0 = np.asarray(h0, dtype=np.float32)
    num_layers = len(layer_outputs)
    blocks, partial, per_layer = [], None, []
    for l, ((n, i), F) in enumerate(zip(block_layout(num_layers, block_size), layer_outputs), start=1):
        if i == 1:
            partial = None
        named = {"h0": h0, "partial": partial}
        named.update({f"b{k + 1}": b for k, b in enumerate(blocks)})
        names = layer_source_names(n, i)
        per_layer.append((names, np.stack([named[x] for x in names])))
        partial = accumulate(partial, F, dtype)
        if i == block_size or l == num_layers:
            blocks.append(partial)
            partial = None
    return per_layer, blocks


def run_schedule_backward(h0, layer_outputs, queries, block_size: int, dtype: str, grad_r,
                          final_query=None, grad_final=None, eps: float = EPS):
    """Backward of ``run_schedule``: every layer's aggregation (and the output
    layer's, if ``final_query`` is given) differentiated, and each source's
    gradient handed to what the source is made of.

    ``grad_r[l-1]`` is dL/dr_l (layer outputs are inputs here, so these are
    independent), ``grad_final`` dL/d(final r).  h_0 is a source of every
    layer; b_k is the sum of block k's layer outputs, so its gradient reaches
    each of them; the partial sum at layer l is the sum of the block's layer
    outputs before l.  Stored sums are rounded to ``dtype`` in the forward; the
    rounding passes gradients through unchanged.

    Returns dict with ``dF`` (list of ``[T, d]``), ``dh0``, ``dw`` (list of
    ``[d]``) and, with ``final_query``, ``dw_final``; all float64.
    """
    num_layers = len(layer_outputs)
    per_layer, blocks = layer_sources(h0, layer_outputs, block_size, dtype)
    layout = block_layout(num_layers, block_size)
    T, d = np.asarray(h0).shape
    dF = [np.zeros((T, d)) for _ in range(num_layers)]
    dh0 = np.zeros((T, d))
    out = {"dw": []}

    def block_members(k):
        return [j for j in range(1, num_layers + 1) if layout[j - 1][0] == k]

    def hand_out(names, dH, layer):
        nonlocal dh0
        for name, g in zip(names, dH):
            if name == "h0":
                dh0 = dh0 + g
            elif name == "partial":          # the block's layers before `layer`
                for j in block_members(layout[layer - 1][0]):
                    if j < layer:
                        dF[j - 1] += g
            else:                            # b_k: every layer of block k
                for j in block_members(int(name[1:])):
                    dF[j - 1] += g

    for l, ((names, H), w, g) in enumerate(zip(per_layer, queries, grad_r), start=1):
        dH, dw = depth_attention_backward(H, w, g, eps)
        out["dw"].append(dw)
        hand_out(names, dH, l)
    if final_query is not None:
        names = ["h0"] + [f"b{k}" for k in range(1, len(blocks) + 1)]
        H = np.stack([np.asarray(h0, np.float32)] + blocks)
        dH, out["dw_final"] = depth_attention_backward(H, final_query, grad_final, eps)
        hand_out(names, dH, None)
    out["dF"] = dF
    out["dh0"] = dh0
    return out
