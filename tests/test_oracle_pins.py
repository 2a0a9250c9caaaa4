"""The oracle against what the pages and the mathematics fix (CPU only).

Also plants plausible mistakes into copies of the oracle's arithmetic and checks
that each one fails at least one pin, so the pins are known to bite.
"""

import numpy as np
import pytest

from oracle import attnres_oracle as orc
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    pin(orc.depth_attention)


# --- planted mistakes (CPU only; the oracle itself is not modified) ----------

def _mutant(keys_fn=None, logits_fn=None, softmax_axis=1, values="raw"):
    def agg(H, w, eps):
        H = np.asarray(H, np.float64)
        w = np.asarray(w, np.float64)
        keys = keys_fn(H, eps) if keys_fn else orc.rmsnorm(H, eps)
        logits = (keys @ w).T
        if logits_fn:
            logits = logits_fn(logits, H)
        a = orc.softmax(logits, axis=softmax_axis)
        V = keys if values == "normalised" else H
        if values == "shifted":
            V = np.roll(H, 1, axis=0)
        r = np.zeros(H.shape[1:])
        for s in range(H.shape[0]):
            r += a[:, s:s + 1] * V[s]
        return r, a
    return agg


MUTANTS = {
    "temperature_1_over_sqrt_d": _mutant(logits_fn=lambda z, H: z / np.sqrt(H.shape[2])),
    "normalised_values": _mutant(values="normalised"),
    "values_off_by_one_source": _mutant(values="shifted"),
    "eps_outside_root": _mutant(keys_fn=lambda H, e: H / (np.sqrt(np.mean(H * H, -1, keepdims=True)) + e)),
    "no_eps": _mutant(keys_fn=lambda H, e: H / np.sqrt(np.mean(H * H, -1, keepdims=True))),
    "sum_not_mean_of_squares": _mutant(keys_fn=lambda H, e: H / np.sqrt(np.sum(H * H, -1, keepdims=True) + e)),
    "norm_over_sources_axis": _mutant(keys_fn=lambda H, e: H / np.sqrt(np.mean(H * H, 0, keepdims=True) + e)),
    "softmax_over_tokens": _mutant(softmax_axis=0),
    "negated_logits": _mutant(logits_fn=lambda z, H: -z),
    "l2_norm_keys": _mutant(keys_fn=lambda H, e: H / np.sqrt(np.sum(H * H, -1, keepdims=True))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    agg = MUTANTS[name]
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(agg)
        except AssertionError as exc:
            failures.append(f"{pin.__name__}: {exc}")
    assert failures, f"planted mistake {name!r} passed every pin"


def test_worked_example_values_are_the_pages():
    """The fixture holds the blog's numbers, and they are a distribution."""
    import json, os
    with open(os.path.join(pins.GOLDEN, "worked_example_four_sources.json")) as f:
        g = json.load(f)
    assert g["depth_weights"] == [0.05, 0.10, 0.70, 0.15]
    assert abs(sum(g["depth_weights"]) - 1.0) < 1e-15
    assert g["residual_coefficients"] == g["depth_weights"]
