"""Linear-layer shapes of the decode workloads (no arithmetic).

Each workload is the set of linear layers one batch-1 decode step applies,
W stored [N_out, K_in]:

* Llama-2-7B: 32 layers of {wqkv 4096->12288, wo 4096->4096,
  w1|w3 fused 4096->22016, w2 11008->4096} plus lm_head 4096->32000.
* Llama-3.1-8B: 32 layers of {wqkv 4096->6144, wo 4096->4096,
  w1|w3 4096->28672, w2 14336->4096} plus lm_head 4096->128256.
* Llama-3.1-70B: 80 layers of {wqkv 8192->10240, wo 8192->8192,
  w1|w3 8192->57344, w2 28672->8192} plus lm_head 8192->128256.
* Mixtral-8x7B MoE: 32 layers of 8 experts, each {w1|w3 4096->28672,
  w2 14336->4096}.

The pages benchmark these model families at batch 1 (gittoolsai "gpt-fast"
README mirror, benchmark table "基准测试" and section "Mixtral 8x7B").
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Model:
    name: str
    dim: int
    qkv: int
    ffn: int
    vocab: int
    layers: int


LLAMA2_7B = Model("llama-2-7b", 4096, 12288, 11008, 32000, 32)
LLAMA31_8B = Model("llama-3.1-8b", 4096, 6144, 14336, 128256, 32)
LLAMA31_70B = Model("llama-3.1-70b", 8192, 10240, 28672, 128256, 80)


@dataclass(frozen=True)
class MoEModel:
    name: str
    dim: int
    ffn: int
    experts: int
    top: int
    layers: int


MIXTRAL_8X7B = MoEModel("mixtral-8x7b", 4096, 14336, 8, 2, 32)

# matrix ids inside one layer (used in seeds)
WQKV, WO, W13, W2, LM_HEAD = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Matrix:
    name: str
    layer: int
    mid: int
    n: int
    k: int

    @property
    def weights(self):
        return self.n * self.k


def layer_matrices(model, layer):
    d = model.dim
    return [
        Matrix("wqkv", layer, WQKV, model.qkv, d),
        Matrix("wo", layer, WO, d, d),
        Matrix("w13", layer, W13, 2 * model.ffn, d),
        Matrix("w2", layer, W2, d, model.ffn),
    ]


def linear_set(model, layers=None):
    """All linears of one decode step: layers x 4 matrices + lm_head."""
    n_layers = model.layers if layers is None else layers
    out = []
    for layer in range(n_layers):
        out += layer_matrices(model, layer)
    out.append(Matrix("lm_head", model.layers, LM_HEAD, model.vocab, model.dim))
    return out


def distinct_shapes(model):
    """One matrix of each distinct shape (layer 0 and lm_head)."""
    return layer_matrices(model, 0) + [Matrix("lm_head", model.layers, LM_HEAD, model.vocab, model.dim)]
