"""The C ABI from a plain C program: depth_wise_attention_block_amd/capi_client,
built with the library, calls attnres_aggregate through include/attnres.h
with the HIP runtime for its device memory -- no Python binding and no torch in
the process that calls the library.  Its results match the oracle to the
parity bar of the other tests."""

import os
import struct
import subprocess

import numpy as np
import pytest
import torch

from depth_wise_attention_block_amd import synth
from tests.gpu_util import compare, host, note, oracle_aggregate

pytestmark = pytest.mark.gpu

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(REPO, "depth_wise_attention_block_amd", "capi_client")


@pytest.mark.parametrize("dtype,S,T,d", [("bf16", 9, 37, 7168), ("bf16", 3, 5, 264), ("f32", 4, 11, 1000),
                                         ("bf16", 20, 3, 520)])
def test_c_client_matches_oracle(tmp_path, dtype, S, T, d):
    note(f"C client {dtype} S={S} T={T} d={d}")
    H = synth.sources(S, T, d, scale=(0.5, 50.0), seed=S + T, dtype=dtype, device="cpu")
    w = synth.query(d, seed=S, device="cpu")
    raw = H.view(torch.int16) if dtype == "bf16" else H
    path_in, path_out = tmp_path / "in.bin", tmp_path / "out.bin"
    path_in.write_bytes(struct.pack("<4i", S, T, d, 0 if dtype == "bf16" else 1) + raw.numpy().tobytes()
                        + w.numpy().astype(np.float32).tobytes())
    r = subprocess.run([CLIENT, str(path_in), str(path_out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    blob = path_out.read_bytes()
    es = 2 if dtype == "bf16" else 4
    assert len(blob) == T * d * es + T * S * 4
    if dtype == "bf16":
        bits = np.frombuffer(blob[: T * d * 2], dtype=np.uint16).astype(np.uint32) << 16
        out = bits.view(np.float32).reshape(T, d)
    else:
        out = np.frombuffer(blob[: T * d * 4], dtype=np.float32).reshape(T, d)
    a = np.frombuffer(blob[T * d * es:], dtype=np.float32).reshape(T, S)
    r_ref, a_ref = oracle_aggregate(host(H), host(w))
    compare(out, a, r_ref, a_ref, dtype == "bf16", f"C client {dtype} S={S}")
