"""CPU oracle for exact softmax attention: test infrastructure only.

Importable by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the library or its Python binding.
"""
from .attention import (attention_fwd_ref, attention_bwd_ref, attention_ref,
                            softmax_vjp_explicit, softmax_vjp_contracted)

__all__ = ["attention_fwd_ref", "attention_bwd_ref", "attention_ref",
           "softmax_vjp_explicit", "softmax_vjp_contracted"]
