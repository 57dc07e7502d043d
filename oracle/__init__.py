"""CPU fp64 oracle for the blocked vocabulary-projection cross-entropy.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never calls it and
shares no code with it.
"""
from .vpce_oracle import (  # noqa: F401
    shard_bounds,
    forward,
    backward,
    dlogits,
    forward_sharded,
    backward_sharded,
    target_logits,
    token_rows,
    vocab_rows_dw,
)
