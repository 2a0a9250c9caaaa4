"""Optional roctx ranges of the schedule drivers (CPU only).  Off by default:
``markers.span`` is one shared no-op context and nothing is loaded.  With
``ATTNRES_ROCTX=1`` the roctx library is loaded and ranges can be pushed and
popped without a profiler attached.  The drivers mark every layer, every
block pass and the output layer, forward and backward."""

import os
import subprocess
import sys

import pytest

from depth_wise_attention_block_amd import markers, schedule
from tests import test_schedule_bytes as tsb

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _probe(env_value):
    env = dict(os.environ)
    env.pop("ATTNRES_ROCTX", None)
    if env_value is not None:
        env["ATTNRES_ROCTX"] = env_value
    code = ("from depth_wise_attention_block_amd import markers\n"
            "with markers.span('layer', 1):\n"
            "    with markers.span('output layer'):\n"
            "        pass\n"
            "print(markers.ENABLED)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=REPO, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout.strip()


def test_off_by_default_and_a_shared_no_op():
    assert _probe(None) == "False"
    assert _probe("0") == "False"
    if not markers.ENABLED:
        assert markers.span("layer", 1) is markers.span("output layer")


@pytest.mark.skipif(not any(os.path.exists(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", n))
                            for n in markers._LIB_NAMES), reason="no roctx library in this image")
def test_enabled_loads_roctx_and_nests():
    assert _probe("1") == "True"


class _Recorder:
    def __init__(self):
        self.names = []

    def __call__(self, kind, index=None):
        self.names.append(kind if index is None else f"{kind} {index}")
        return markers._NULL


def _spans(run):
    rec = _Recorder()
    saved = markers.span
    markers.span = rec
    try:
        run()
    finally:
        markers.span = saved
    return rec.names


def test_forward_spans_every_layer_block_pass_and_the_output_layer():
    names = _spans(lambda: tsb._run("two_phase", T=1, d=8))
    assert [n for n in names if n.startswith("layer ")] == [f"layer {l}" for l in range(1, 94)]
    assert [n for n in names if n.startswith("inter-block")] == [f"inter-block pass of block {b}" for b in range(3, 9)]
    assert names[-1] == "output layer"


def test_backward_spans_every_layer_and_block_pass():
    names = _spans(lambda: tsb._run_backward(1, 8, True))
    assert names[0] == "output layer backward"
    assert [n for n in names if n.startswith("layer backward")] == [f"layer backward {l}" for l in range(93, 0, -1)]
    assert [n for n in names if n.startswith("gradient rows")] == [f"gradient rows of block {b}" for b in range(8, 0, -1)]
    assert [n for n in names if n.startswith("partial sums")] == [f"partial sums of block {b}" for b in range(8, 0, -1)]
