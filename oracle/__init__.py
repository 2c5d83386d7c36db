"""Float64 CPU oracle of the decode path and of the prefill ground truth --
test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library or its binding.
"""
from .seer_oracle import *  # noqa: F401,F403
from .seer_oracle import topk_budget_blocks, sparse_decode_pair  # noqa: F401
from .prefill_gt import (group_ground_truth, pooled_attention_map,  # noqa: F401
                         prefill_attention, prefill_group)
