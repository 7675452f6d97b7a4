"""Pin the oracle's storage formats to the pages' benchmark tables (CPU only).

The pages print tokens/s next to "memory bandwidth (GB/s)" for batch-1 decode
(gittoolsai "gpt-fast" README mirror, tables "基准测试" and "AMD"; rows are
stored in tests/golden/pages_benchmark_rows.json).  Their ratio is the bytes
read per token.  Rebuilding that figure from the model shapes and the bytes
per weight the oracle's quantizers actually emit reproduces the printed
numbers: int8 stores one byte per weight plus one bf16 per output row, int4
G=32 stores 0.625 byte per weight (a 4-bit code plus a bf16 scale and zero
per 32 weights).  A format with another size (fp32 scales, an int zero-point
byte, a group of 64) misses the rows by several percent.

Model shapes: Llama-2-7B, Llama-3.1-8B and Llama-3.1-70B as in ``synth``;
Llama-2-70B shares Llama-3.1-70B's dimensions with a 32000-entry vocabulary.
Each layer adds two bf16 norm vectors and the model one final norm.  The
Llama-2 rows count the bf16 token embedding, the Llama-3.1 rows do not (the
field ``embedding_counted``).
"""

import json
import os

import numpy as np
import pytest

from oracle.quant import quantize_int8, quantize_int4g32
from oracle.bf16 import round_f32_to_bf16
from synth.configs import LLAMA2_7B, LLAMA2_70B, LLAMA31_8B, LLAMA31_70B, linear_set
MODELS = {m.name: m for m in (LLAMA2_7B, LLAMA31_8B, LLAMA31_70B, LLAMA2_70B)}
HERE = os.path.dirname(os.path.abspath(__file__))


def _format_costs():
    """(bytes per weight, bytes per output row) measured on oracle outputs."""
    rng = np.random.default_rng(41)
    n, k = 64, 256
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    packed, sz = quantize_int4g32(w)
    wb = round_f32_to_bf16(w)
    return {
        "int8": (q.nbytes / (n * k), s.nbytes / n),
        "int4g32": ((packed.nbytes + sz.nbytes) / (n * k), 0.0),
        "bf16": (wb.nbytes / (n * k), 0.0),
    }


def model_bytes(model, fmt, embedding_counted, costs):
    per_w, per_row = costs[fmt]
    mats = linear_set(model)
    linear = sum(m.weights for m in mats) * per_w + sum(m.n for m in mats) * per_row
    norms = (2 * model.layers + 1) * model.dim * 2
    emb = model.vocab * model.dim * 2 if embedding_counted else 0
    return linear + norms + emb


def test_format_costs_are_what_the_tables_imply():
    c = _format_costs()
    assert c["int8"] == (1.0, 2.0)
    assert c["int4g32"] == (0.625, 0.0)
    assert c["bf16"] == (2.0, 0.0)


with open(os.path.join(HERE, "golden", "pages_benchmark_rows.json")) as fh:
    ROWS = json.load(fh)["rows"]


@pytest.mark.parametrize("row", ROWS, ids=lambda r: f"{r['model']}-{r['format']}-{r['hw']}")
def test_bytes_per_token_match_printed_bandwidth(row):
    costs = _format_costs()
    printed = row["gb_s"] / row["tok_s"] * 1e9
    modelled = model_bytes(MODELS[row["model"]], row["format"], row["embedding_counted"], costs)
    tol = 0.015 if "note" in row else 0.005
    assert abs(modelled / printed - 1) < tol, (modelled, printed)


def test_a_different_int4_format_would_not_match():
    # 4-bit codes with fp32 scale+zero per group of 32 (0.75 B/weight) misses by >10%
    costs = _format_costs()
    costs["int4g32"] = (0.75, 0.0)
    row = next(r for r in ROWS if r["model"] == "llama-2-70b" and r["format"] == "int4g32")
    printed = row["gb_s"] / row["tok_s"] * 1e9
    assert abs(model_bytes(LLAMA2_70B, "int4g32", True, costs) / printed - 1) > 0.10
