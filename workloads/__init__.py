"""Seeded synthetic inputs for DMS attention workloads.

This package draws random numbers and nothing else: it holds none of the
method's arithmetic (no decisions, no masks, no attention).  Both the HIP path
and the float64 oracle receive the tensors it returns.
"""

from .configs import WORKLOADS, Workload, get  # noqa: F401
from .synth import (  # noqa: F401
    logit_mean_for_rate,
    logistic_noise,
    decode_step_inputs,
    prompt_chunk_inputs,
    prefill_inputs,
    unit_eviction_rates,
)
