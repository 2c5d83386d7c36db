"""Float64 CPU oracle of the decode path -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library or its binding.
"""
from .seer_oracle import *  # noqa: F401,F403
from .seer_oracle import topk_budget_blocks, sparse_decode_pair  # noqa: F401
