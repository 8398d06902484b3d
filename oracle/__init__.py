"""CPU oracle of the RG-LRU temporal branch (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
package; the HIP library never does.
"""
from .rglru_oracle import (round_io, sigmoid, log_sigmoid, gates, conv1d_causal4,  # noqa: F401
                           forward, decode_step, backward, gelu, block_forward,
                           gated_mlp_forward, HEAD_DIM, rope, local_mqa_attention,
                           local_mqa_forward, local_mqa_decode_step)
