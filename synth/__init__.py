"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This package draws random tensors and nothing else: it holds none of the KDA
arithmetic, and neither the oracle nor the HIP path lives here.
"""

from .inputs import WORKLOADS, decode_inputs, gate_inputs, prefill_inputs, workload_inputs

__all__ = ["WORKLOADS", "decode_inputs", "gate_inputs", "prefill_inputs", "workload_inputs"]
