"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package holds shapes and random-number plumbing only: no quantization,
no dequantization, no matvec arithmetic.  Both the CPU oracle and the HIP
library consume what it produces; neither is imported here.
"""

from .configs import (  # noqa: F401
    LLAMA2_7B, LLAMA31_8B, LLAMA31_70B, MIXTRAL_8X7B,
    linear_set, Matrix,
)
from .gen import (  # noqa: F401
    seed_for, host_normal, host_bf16_normal, host_logits,
)
