"""CPU oracle (test infrastructure only; never on the product path).

Importable only from tests, the smoke check and the bench's CPU-baseline leg.
"""

from . import fp8
from .attention import allowed_mask, attention_bwd, attention_fwd, attention_rows, bf16_bits_to_f64

__all__ = ["allowed_mask", "attention_bwd", "attention_fwd", "attention_rows", "bf16_bits_to_f64", "fp8"]
