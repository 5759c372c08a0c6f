"""CPU fp64 oracle of the dense attention forward (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import
this package; it shares no code with the HIP path.
"""
from .attention_ref import attention, attention_probs, attention_rows, sigma_of
from .online_model import online_attention

__all__ = ["attention", "attention_probs", "attention_rows", "online_attention", "sigma_of"]
