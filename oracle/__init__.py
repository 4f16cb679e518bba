"""Float64 CPU oracle for SANA's ReLU linear attention (test infrastructure only).

Importers allowed: the test suite, the smoke check and the CPU-baseline leg of
the benchmark.  The product path never imports this package.
"""

from .linattn_oracle import (  # noqa: F401
    feature_map,
    rope3d_angles,
    rotate_pairs,
    kv_state,
    apply_state,
    linattn,
    state_update,
    block_forward,
    block_causal,
    brute_force,
    backward,
    temporal_conv3,
    round_bf16,
    projected_apply,
    projected_kv_state,
)
