"""Seeded synthetic workloads (inputs only, none of the method's arithmetic)."""
from .synth import WORKLOADS, Workload, make_inputs, append_token, draw_seq_lens  # noqa: F401
from .synth import PREFILL_WORKLOADS, PrefillWorkload, make_prefill_inputs  # noqa: F401
