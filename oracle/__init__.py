"""CPU oracle for weight-only quantized decode matvecs.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
bench's CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes (plain, slow, obviously correct; fp64 unless a step fixes
another precision):

* ``bf16``    -- fp32 -> bf16 round-to-nearest-even and exact bf16 decoding.
* ``quant``   -- int8 per-output-row symmetric quantization and int4
                 asymmetric quantization with groups of 32 inputs, bf16
                 scale and zero, two codes per byte.
* ``matvec``  -- the dequantized matvec y = x . W^T in fp64 (bf16, int8,
                 int4 G=32 weights; one token or a few speculative tokens).
* ``moe``     -- top-2 routing with renormalised gates over 8 experts and
                 the SwiGLU expert FFN built from two quantized GEMVs.

Sources.  The pages describe gpt-fast, a PyTorch decode engine: int8 and
int4 weight-only quantization with a group-size knob (gittoolsai "gpt-fast"
README mirror, section "量化 / Int8 仅权重量化, Int4 仅权重量化"; awesome-
repositories "meta-pytorch/gpt-fast", tag "Grouped Quantization"),
speculative decoding where a larger model verifies the draft's tokens
(onegen.ai "Efficiently implementing the Mixtral 8x7B model with gpt-fast",
section "Key Features"), and Mixtral 8x7B sparse MoE (gittoolsai mirror,
section "Mixtral 8x7B").  The pages do not state the quantization formulas,
the rounding rule, the packing, nor the expert FFN; each function below
names the reading it takes where the pages are silent.

Parity pins.  Every function here is pinned by tests that do not re-type its
formula: closed forms, brute-force argmin over all codes, exact rational
arithmetic, invariants and the storage cost the pages' benchmark tables
imply.  Nothing here is "parity unpinned" except where a function's
docstring says so.
"""

from . import bf16, quant, matvec, moe  # noqa: F401
