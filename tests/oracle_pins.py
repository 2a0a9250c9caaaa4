"""Checks that pin an aggregation ``agg(H, w, eps) -> (r, a)`` to facts that do not
come from the aggregation itself.

Each ``pin_*`` function raises ``AssertionError`` when ``agg`` disagrees with
the fact it encodes.  The oracle must pass all of them; every planted mistake
in ``test_oracle_pins.py`` must fail at least one.  Facts used:

* the worked example of "Kimi K3技术详解系列（二）：AttnRes 与 Stable LatentMoE"
  §2.1 (depth weights 0.05/0.10/0.70/0.15 and the matching residual), rebuilt
  by solving for a pseudo-query with torch's own RMSNorm;
* a library reduction: ``torch.nn.functional.rms_norm`` for the keys and
  ``scaled_dot_product_attention`` (scale 1) for softmax and weighted sum;
* closed forms: one source, a zero query (the uniform mixer of llm-atlas's
  uniform-mixer study), identical sources, two sources (a logistic), a huge query
  (one-hot);
* invariants: weights non-negative summing to one (§2 of the blog above),
  keys blind to a positive rescaling (kimi.papertok.ai ch. 0 §0.11),
  permutation equivariance;
* 50-digit brute force on tiny inputs.
"""

from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np
import torch
import torch.nn.functional as F
from scipy.special import expit

from depth_wise_attention_block_amd import synth

EPS = 1e-5
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(x, y, rtol, atol=0.0, what=""):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, f"{what}: shape {x.shape} vs {y.shape}"
    err = np.max(np.abs(x - y)) if x.size else 0.0
    lim = atol + rtol * (np.max(np.abs(y)) if y.size else 0.0)
    assert err <= lim, f"{what}: max error {err:.3e} > {lim:.3e}"


def library_keys(H, eps=EPS):
    """Keys by torch's RMSNorm (no gain), float64."""
    Ht = torch.as_tensor(np.asarray(H, np.float64))
    return F.rms_norm(Ht, (Ht.shape[-1],), eps=eps).numpy()


def library_reference(H, w, eps=EPS):
    """Residual and weights by torch's RMSNorm + scaled_dot_product_attention."""
    Ht = torch.as_tensor(np.asarray(H, np.float64))
    S, T, d = Ht.shape
    keys = F.rms_norm(Ht, (d,), eps=eps).permute(1, 0, 2).contiguous()     # [T, S, d]
    q = torch.as_tensor(np.asarray(w, np.float64)).view(1, 1, d).expand(T, 1, d).contiguous()
    values = Ht.permute(1, 0, 2).contiguous()
    r = F.scaled_dot_product_attention(q, keys, values, scale=1.0)[:, 0, :]
    onehot = torch.eye(S, dtype=torch.float64).expand(T, S, S).contiguous()
    a = F.scaled_dot_product_attention(q, keys, onehot, scale=1.0)[:, 0, :]
    return r.numpy(), a.numpy()


def worked_example_inputs(d=256, tokens=8, seed=0, scale=(0.1, 10.0), dtype="f32"):
    """Sources h0..h3 and a pseudo-query that gives every token the depth weights
    of the blog's §2.1 walk-through.

    The keys come from torch's RMSNorm; the query is the minimum-norm solution
    of ``keys . w = ln(weights)`` over all tokens (4*tokens equations, d
    unknowns), so softmax of the logits is exactly the target.  Returns the
    sources (float32 values, already in ``dtype``'s precision), w (float64)
    and the target weights.
    """
    with open(os.path.join(GOLDEN, "worked_example_four_sources.json")) as f:
        target = np.array(json.load(f)["depth_weights"], np.float64)
    H = synth.sources(4, tokens, d, scale=scale, seed=seed, dtype=dtype).float().numpy()
    K = library_keys(H)                                      # [4, T, d]
    A = K.transpose(1, 0, 2).reshape(4 * tokens, d)          # token-major equations
    rhs = np.tile(np.log(target), tokens)
    w = np.linalg.lstsq(A, rhs, rcond=None)[0]
    return H, w, target


def pin_worked_example(agg, rtol=1e-12):
    H, w, target = worked_example_inputs()
    r, a = agg(H, w, EPS)
    _close(a, np.broadcast_to(target, a.shape), rtol=0, atol=rtol, what="worked-example weights")
    expect = sum(c * H[i].astype(np.float64) for i, c in enumerate(target))
    _close(r, expect, rtol=rtol, what="worked-example residual")


def pin_library(agg, seed=1):
    # scales reach down to 1e-3, so some source has mean square near eps:
    # that separates eps-inside-the-root from other placements.
    H = synth.sources(6, 16, 64, scale=(1e-3, 10.0), seed=seed, dtype="f32").double().numpy()
    H[2] *= 3e-3 / np.sqrt(np.mean(H[2] ** 2))            # mean square 9e-6 ~ eps
    w = synth.query(64, seed=seed).double().numpy()
    r, a = agg(H, w, EPS)
    r_lib, a_lib = library_reference(H, w, EPS)
    _close(a, a_lib, rtol=0, atol=1e-12, what="weights vs library")
    _close(r, r_lib, rtol=1e-12, what="residual vs library")


def pin_closed_forms(agg, seed=2):
    rng = np.random.default_rng(seed)
    S, T, d = 5, 7, 32
    H = rng.normal(size=(S, T, d)) * rng.uniform(0.5, 4.0, size=(S, 1, 1))
    w = rng.normal(scale=2 / math.sqrt(d), size=d)
    # one source: weight 1, residual is that source, exactly
    r, a = agg(H[:1], w, EPS)
    assert np.array_equal(a, np.ones((T, 1))), "S=1 weight must be exactly 1"
    assert np.array_equal(r, H[0]), "S=1 residual must be h0 exactly"
    # zero query: the uniform mixer, weights 1/S and the mean of the sources
    r, a = agg(H, np.zeros(d), EPS)
    _close(a, np.full((T, S), 1.0 / S), rtol=0, atol=1e-15, what="zero-query weights")
    _close(r, np.mean(H, axis=0), rtol=1e-14, what="zero-query residual")
    # identical sources: uniform weights, residual equals the source
    same = np.repeat(H[:1], 4, axis=0)
    r, a = agg(same, w, EPS)
    _close(a, np.full((T, 4), 0.25), rtol=0, atol=1e-15, what="identical-source weights")
    _close(r, H[0], rtol=1e-14, what="identical-source residual")
    # two sources: a_1 = logistic(z_1 - z_0)
    K = library_keys(H[:2])
    z = K @ w                                            # [2, T]
    r, a = agg(H[:2], w, EPS)
    _close(a[:, 1], expit(z[1] - z[0]), rtol=0, atol=1e-14, what="two-source logistic")
    _close(a[:, 0], expit(z[0] - z[1]), rtol=0, atol=1e-14, what="two-source logistic")
    # huge query: one-hot on the largest logit, no overflow
    big = 1e3 * w
    r, a = agg(H, big, EPS)
    zb = library_keys(H) @ big                           # [S, T]
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(r)), "overflow with a large query"
    top = np.argmax(zb, axis=0)
    _close(a, np.eye(S)[top], rtol=0, atol=1e-12, what="one-hot weights")
    _close(r, H[top, np.arange(T)], rtol=1e-12, what="one-hot residual")


def pin_invariants(agg, seed=3):
    rng = np.random.default_rng(seed)
    S, T, d = 6, 9, 48
    H = rng.normal(size=(S, T, d)) * rng.uniform(0.5, 4.0, size=(S, 1, 1))
    w = rng.normal(scale=2 / math.sqrt(d), size=d)
    r, a = agg(H, w, EPS)
    assert np.all(a >= 0), "negative depth weight"
    _close(a.sum(axis=1), np.ones(T), rtol=0, atol=1e-14, what="weights sum")
    # rescaling a source by c > 0 leaves its key (hence every weight) unchanged up
    # to eps, and moves the residual by a_s (c - 1) H_s
    c, s = 7.0, 3
    H2 = H.copy()
    H2[s] *= c
    r2, a2 = agg(H2, w, EPS)
    _close(a2, a, rtol=0, atol=2e-4, what="rescaled-source weights")
    _close(r2, r + a[:, s:s + 1] * (c - 1) * H[s], rtol=2e-4, what="rescaled-source residual")
    # permuting the sources permutes the weights and keeps the residual
    perm = rng.permutation(S)
    r3, a3 = agg(H[perm], w, EPS)
    _close(a3, a[:, perm], rtol=0, atol=1e-14, what="permuted weights")
    _close(r3, r, rtol=1e-13, what="permuted residual")


def _mp_reference(H, w, eps, digits=50):
    """The definition evaluated in 50-digit arithmetic, term by term."""
    mpmath.mp.dps = digits
    S, T, d = H.shape
    r = np.zeros((T, d))
    a = np.zeros((T, S))
    for t in range(T):
        z = []
        for s in range(S):
            row = [mpmath.mpf(float(v)) for v in H[s, t]]
            ms = mpmath.fsum(v * v for v in row) / d
            inv = 1 / mpmath.sqrt(ms + mpmath.mpf(eps))
            z.append(mpmath.fsum(mpmath.mpf(float(w[j])) * row[j] * inv for j in range(d)))
        e = [mpmath.exp(zz) for zz in z]
        tot = mpmath.fsum(e)
        for s in range(S):
            a[t, s] = float(e[s] / tot)
        for j in range(d):
            r[t, j] = float(mpmath.fsum(e[s] / tot * mpmath.mpf(float(H[s, t, j])) for s in range(S)))
    return r, a


def pin_bruteforce(agg, seed=4):
    rng = np.random.default_rng(seed)
    for S, T, d in ((1, 2, 4), (3, 3, 8), (9, 2, 16)):
        H = rng.normal(size=(S, T, d)) * rng.uniform(0.01, 10.0, size=(S, 1, 1))
        w = rng.normal(scale=2.0, size=d)
        r, a = agg(H, w, EPS)
        r_mp, a_mp = _mp_reference(H, w, EPS)
        _close(a, a_mp, rtol=0, atol=1e-12, what=f"brute-force weights S={S}")
        _close(r, r_mp, rtol=1e-12, what=f"brute-force residual S={S}")


ALL_PINS = (pin_worked_example, pin_library, pin_closed_forms, pin_invariants, pin_bruteforce)


# ----------------------------------------------------------------------------
# Backward pins: ``bwd(H, w, g, eps) -> (dH, dw)``, the gradients of
# ``sum(g * r)``.  Facts used: torch autograd through the library reduction
# above; central finite differences (Richardson-extrapolated) of the forward;
# closed forms (one source: the gradient passes through unchanged; a zero
# query or identical sources: every source gets g / S); the rescaling
# invariant (keys blind to a positive rescaling, so d/dc L(c H_s) = a_s g.H_s
# up to eps); permutation equivariance.
# ----------------------------------------------------------------------------

def library_backward(H, w, g, eps=EPS):
    """dL/dH and dL/dw of L = sum(g * r) by autograd through rms_norm + sdpa."""
    Ht = torch.tensor(np.asarray(H, np.float64), requires_grad=True)
    wt = torch.tensor(np.asarray(w, np.float64), requires_grad=True)
    S, T, d = Ht.shape
    keys = F.rms_norm(Ht, (d,), eps=eps).permute(1, 0, 2)
    q = wt.view(1, 1, d).expand(T, 1, d)
    r = F.scaled_dot_product_attention(q, keys, Ht.permute(1, 0, 2), scale=1.0)[:, 0, :]
    (r * torch.as_tensor(np.asarray(g, np.float64))).sum().backward()
    return Ht.grad.numpy(), wt.grad.numpy()


def pin_backward_library(bwd, seed=11):
    H = synth.sources(6, 16, 64, scale=(1e-3, 10.0), seed=seed, dtype="f32").double().numpy()
    H[2] *= 3e-3 / np.sqrt(np.mean(H[2] ** 2))            # mean square near eps
    w = synth.query(64, seed=seed).double().numpy()
    g = np.random.default_rng(seed).normal(size=(16, 64))
    dH, dw = bwd(H, w, g, EPS)
    dH_lib, dw_lib = library_backward(H, w, g, EPS)
    _close(dH, dH_lib, rtol=1e-11, what="dH vs autograd")
    _close(dw, dw_lib, rtol=1e-11, what="dw vs autograd")


def _loss(H, w, g, eps):
    from oracle import attnres_oracle as orc   # the forward, pinned by the pins above
    r, _ = orc.depth_attention(H, w, eps)
    return float(np.sum(g * r))


def pin_backward_finite_difference(bwd, seed=12):
    rng = np.random.default_rng(seed)
    for S, T, d in ((1, 2, 4), (3, 2, 8), (9, 2, 8)):
        H = rng.normal(size=(S, T, d)) * rng.uniform(0.3, 3.0, size=(S, 1, 1))
        w = rng.normal(scale=1.0, size=d)
        g = rng.normal(size=(T, d))
        dH, dw = bwd(H, w, g, EPS)
        for trial in range(4):
            V = rng.normal(size=H.shape)
            v = rng.normal(size=d)

            def D(h):
                return (_loss(H + h * V, w + h * v, g, EPS) - _loss(H - h * V, w - h * v, g, EPS)) / (2 * h)
            fd = (4 * D(5e-4) - D(1e-3)) / 3                  # Richardson: error O(h^4)
            an = float(np.sum(dH * V) + np.sum(dw * v))
            assert abs(fd - an) <= 1e-8 * max(1.0, abs(fd)), f"S={S} direction {trial}: {an} vs {fd}"


def pin_backward_closed_forms(bwd, seed=13):
    rng = np.random.default_rng(seed)
    S, T, d = 5, 7, 32
    H = rng.normal(size=(S, T, d)) * rng.uniform(0.5, 4.0, size=(S, 1, 1))
    w = rng.normal(scale=2 / math.sqrt(d), size=d)
    g = rng.normal(size=(T, d))
    # one source: r = h0, so dH = g exactly and the query gets nothing
    dH, dw = bwd(H[:1], w, g, EPS)
    assert np.array_equal(dH[0], g), "S=1: the gradient must pass through unchanged"
    assert np.array_equal(dw, np.zeros(d)), "S=1: the query gradient must be zero"
    # zero query: uniform weights, each source gets g / S (the key path carries w = 0)
    dH, dw = bwd(H, np.zeros(d), g, EPS)
    _close(dH, np.broadcast_to(g / S, dH.shape), rtol=1e-14, what="zero-query dH")
    # identical sources: uniform weights, equal scores, no softmax gradient
    same = np.repeat(H[:1], 4, axis=0)
    dH, dw = bwd(same, w, g, EPS)
    _close(dH, np.broadcast_to(g / 4, dH.shape), rtol=1e-13, what="identical-source dH")
    _close(dw, np.zeros(d), rtol=0, atol=1e-12 * np.max(np.abs(g)) * np.max(np.abs(H)), what="identical-source dw")


def pin_backward_invariants(bwd, seed=14):
    rng = np.random.default_rng(seed)
    S, T, d = 6, 9, 48
    H = rng.normal(size=(S, T, d)) * rng.uniform(0.5, 4.0, size=(S, 1, 1))
    w = rng.normal(scale=2 / math.sqrt(d), size=d)
    g = rng.normal(size=(T, d))
    from oracle import attnres_oracle as orc
    _, a = orc.depth_attention(H, w, EPS)
    dH, dw = bwd(H, w, g, EPS)
    # keys are blind to a positive rescaling of a source (up to eps), so along
    # H_s the loss changes only through the value: H_s . dH_s = a_s g . H_s
    lhs = np.sum(H * dH, axis=-1)                               # [S, T]
    rhs = (a.T * np.sum(g[None] * H, axis=-1))                  # [S, T]
    _close(lhs, rhs, rtol=1e-4, what="rescaling invariant")
    # permuting the sources permutes dH and leaves dw
    perm = rng.permutation(S)
    dH2, dw2 = bwd(H[perm], w, g, EPS)
    _close(dH2, dH[perm], rtol=1e-13, what="permuted dH")
    _close(dw2, dw, rtol=1e-13, what="permuted dw")


BACKWARD_PINS = (pin_backward_library, pin_backward_finite_difference, pin_backward_closed_forms,
                 pin_backward_invariants)


def library_backward_per_source(H, w, g, eps=EPS):
    """Each source's share of dL/dw by autograd: one copy of the query per source
    logit, keys from torch ``rms_norm``, softmax and weighted sum from torch."""
    Ht = torch.tensor(np.asarray(H, np.float64))
    S, T, d = Ht.shape
    Wt = torch.tensor(np.repeat(np.asarray(w, np.float64)[None], S, axis=0), requires_grad=True)   # [S, d]
    keys = F.rms_norm(Ht, (d,), eps=eps)                                    # [S, T, d]
    z = torch.stack([keys[s] @ Wt[s] for s in range(S)], dim=1)             # [T, S]
    a = torch.softmax(z, dim=1)
    r = sum(a[:, s:s + 1] * Ht[s] for s in range(S))
    (r * torch.as_tensor(np.asarray(g, np.float64))).sum().backward()
    return Wt.grad.numpy()


def pin_backward_per_source(bwd_src, seed=15):
    """``bwd_src(H, w, g, eps) -> (dw, dw_src)``: the per-source shares equal
    autograd through per-source query copies and sum to dL/dw."""
    H = synth.sources(5, 12, 48, scale=(0.01, 20.0), seed=seed, dtype="f32").double().numpy()
    w = synth.query(48, seed=seed).double().numpy()
    g = np.random.default_rng(seed).normal(size=(12, 48))
    dw, dw_src = bwd_src(H, w, g, EPS)
    _close(dw_src, library_backward_per_source(H, w, g, EPS), rtol=1e-11, what="per-source dw vs autograd")
    _close(dw_src.sum(axis=0), dw, rtol=1e-12, what="per-source shares sum to dw")
