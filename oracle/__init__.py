"""CPU oracle for the Block AttnRes depth aggregation (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the product path never does.
"""

from .attnres_oracle import (EPS, accumulate, bf16_bits_to_f32, bf16_round,  # noqa: F401
                             block_layout, depth_attention, f32_to_bf16_bits,
                             layer_source_names, rmsnorm, run_full_schedule, run_schedule,
                             softmax)
