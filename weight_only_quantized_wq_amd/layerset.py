"""Decode-step linear sets resident in HBM, driven through libwq.

A batch-1 decode step applies every linear layer of the model once (the
pages' benchmark protocol: gittoolsai "gpt-fast" README mirror, section
"基准测试", batch size 1).  ``LayerSet`` holds one model's linears quantized in
device memory and ``step()`` launches one matvec per matrix, back to back on
one stream, each with its own activation vector; nothing is chained between
matrices (attention, norms and the embedding are not on this path).

Weights are produced on the device by a caller-supplied generator (fp32),
quantized there by the library's own quantizer and the fp32 copy freed, so a
70B-parameter set never passes through host memory.

Algorithmic bytes per matrix (what the product must move): the stored
weights (bf16 2 B/weight; int8 1 B/weight + 2 B/row; int4 G=32 0.625
B/weight), the bf16 activations read (2 B per input per token) and the bf16
outputs written (2 B per output per token).
"""

import torch

from . import _binding as wq

FORMATS = ("bf16", "int8", "int4g32", "int4g64", "int4g128", "int4g256", "int4pc")


def int4_group(fmt, k):
    """Group size of an int4 format for rows of k inputs (``int4g<G>``: G;
    ``int4pc``, one group per row: k); 0 for the other formats."""
    if fmt == "int4pc":
        return k
    return int(fmt[5:]) if fmt.startswith("int4g") else 0


def weight_bytes(fmt, n, k):
    if fmt == "bf16":
        return 2 * n * k
    if fmt == "int8":
        return n * k + 2 * n
    if int4_group(fmt, k):
        return n * k // 2 + (k // int4_group(fmt, k)) * 4 * n
    raise ValueError(fmt)


def matrix_bytes(fmt, n, k, m=1):
    return weight_bytes(fmt, n, k) + 2 * m * k + 2 * m * n


class QuantMatrix:
    """One quantized linear in device memory plus its activation/output buffers."""

    def __init__(self, fmt, n, k, w32, x, m=1):
        self.fmt, self.n, self.k, self.m = fmt, n, k, m
        dev = w32.device
        if fmt == "bf16":
            self.w = w32.to(torch.bfloat16).view(torch.int16).contiguous()
            self.aux = None
        elif fmt == "int8":
            self.w = torch.empty((n, k), dtype=torch.int8, device=dev)
            self.aux = torch.empty((n,), dtype=torch.int16, device=dev)
            wq.wq_quantize_int8(w32, n, k, self.w, self.aux)
        elif int4_group(fmt, k):
            g = int4_group(fmt, k)
            self.w = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
            self.aux = torch.empty((n, k // g, 2), dtype=torch.int16, device=dev)
            wq.wq_quantize_int4(w32, n, k, g, self.w, self.aux)
        else:
            raise ValueError(fmt)
        self.x = x
        self.y16 = torch.empty((m, n), dtype=torch.int16, device=dev)
        self.y32 = None
        self.bytes = matrix_bytes(fmt, n, k, m)

    def launch(self, stream=None, y32=None):
        y16 = self.y16
        if self.fmt == "bf16":
            wq.wq_gemv_bf16(self.x, self.w, self.n, self.k, y32, y16, stream)
        elif self.fmt == "int8" and self.m == 1:
            wq.wq_gemv_int8(self.x, self.w, self.aux, self.n, self.k, y32, y16, stream)
        elif self.fmt == "int8":
            wq.wq_gemm_smallM_int8(self.x, self.m, self.w, self.aux, self.n, self.k, y32, y16, stream)
        elif self.m == 1:
            wq.wq_gemv_int4(self.x, self.w, self.aux, self.n, self.k, int4_group(self.fmt, self.k), y32, y16, stream)
        else:
            wq.wq_gemm_smallM_int4(self.x, self.m, self.w, self.aux, self.n, self.k, int4_group(self.fmt, self.k),
                                   y32, y16, stream)


class LayerSet:
    """All linears of one decode step for a list of ``synth.configs.Matrix``.

    gen_w(n, k, matrix) -> fp32 [n, k] device tensor; gen_x(m, k, matrix) ->
    bf16 [m, k] (or [k]) device tensor.
    """

    def __init__(self, matrices, fmt, gen_w, gen_x, m=1, device="cuda"):
        self.fmt, self.m = fmt, m
        self.mats = []
        for mat in matrices:
            w32 = gen_w(mat.n, mat.k, mat)
            x = gen_x(m, mat.k, mat).contiguous()
            self.mats.append(QuantMatrix(fmt, mat.n, mat.k, w32, x, m))
            del w32
        torch.cuda.synchronize(device)
        self.bytes = sum(q.bytes for q in self.mats)

    def step(self, stream=None):
        """One decode step as one launch per matrix."""
        for q in self.mats:
            q.launch(stream)

    def prepare_fused(self, with_f32=False):
        """Plans the whole step as one persistent launch (wq_decode_step_*)."""
        dev = self.mats[0].w.device
        if with_f32:
            for q in self.mats:
                if q.y32 is None:
                    q.y32 = torch.empty((q.m, q.n), dtype=torch.float32, device=dev)
        nbytes = wq.wq_decode_step_workspace_bytes(len(self.mats))
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        mats = [(q.x, q.w, q.aux, q.n, q.k, q.y32, q.y16) for q in self.mats]
        self.plan = wq.wq_decode_step_prepare(self.fmt, self.m, mats, self.workspace)
        return self.plan

    def step_fused(self, stream=None):
        """One decode step as one persistent launch (call prepare_fused first)."""
        wq.wq_decode_step_run(self.plan, stream)


def moe_layer_bytes(dim, f, top=2):
    """Bytes one MoE decode layer must move: the `top` selected experts' int8
    W13 [2f, dim] and W2 [dim, f] with their bf16 row scales, the bf16
    activation and output, the 8 fp32 logits and the fp32 SwiGLU workspace
    written once and read once."""
    experts = top * (2 * f * dim + 2 * 2 * f + dim * f + 2 * dim)
    return experts + 2 * dim + 2 * dim + 8 * 4 + 2 * (top * f * 4)


class MoELayerSet:
    """Top-2 MoE decode layers (int8 experts) resident in device memory.

    gen_w(rows, cols, key) -> fp32 device tensor; gen_x(dim, layer) -> bf16
    [dim]; gen_logits(e, layer) -> fp32 [e] device tensor.  key =
    (layer, expert, 0 for w1|w3 or 1 for w2).
    """

    def __init__(self, dim, f, experts, layers, gen_w, gen_x, gen_logits, device="cuda"):
        self.dim, self.f, self.e = dim, f, experts
        self.layers = []
        for layer in range(layers):
            w13 = torch.empty((experts, 2 * f, dim), dtype=torch.int8, device=device)
            s13 = torch.empty((experts, 2 * f), dtype=torch.int16, device=device)
            w2 = torch.empty((experts, dim, f), dtype=torch.int8, device=device)
            s2 = torch.empty((experts, dim), dtype=torch.int16, device=device)
            for e in range(experts):
                w = gen_w(2 * f, dim, (layer, e, 0))
                wq.wq_quantize_int8(w, 2 * f, dim, w13[e], s13[e])
                del w
                w = gen_w(dim, f, (layer, e, 1))
                wq.wq_quantize_int8(w, dim, f, w2[e], s2[e])
                del w
            self.layers.append(dict(
                w13=w13, s13=s13, w2=w2, s2=s2,
                x=gen_x(dim, layer).contiguous(), logits=gen_logits(experts, layer).contiguous(),
                work=torch.empty(2 * f, dtype=torch.float32, device=device),
                y16=torch.empty(dim, dtype=torch.int16, device=device)))
        torch.cuda.synchronize(device)
        self.bytes = layers * moe_layer_bytes(dim, f)

    def launch_layer(self, i, stream=None, y32=None, sel=None, gates=None):
        L = self.layers[i]
        wq.moe_top2_gemv(L["x"], L["logits"], self.e, L["w13"], L["s13"], L["w2"], L["s2"], self.dim, self.f,
                         L["work"], y32, L["y16"], sel, gates, stream)

    def step(self, stream=None):
        """One decode step as one moe_top2_gemv call (two launches) per layer."""
        for i in range(len(self.layers)):
            self.launch_layer(i, stream)

    def prepare_fused(self, with_f32=False, with_sel=False):
        """Plans all layers as two persistent launches (wq_moe_step_*)."""
        dev = self.layers[0]["x"].device
        for L in self.layers:
            if with_f32 and L.get("y32") is None:
                L["y32"] = torch.empty(self.dim, dtype=torch.float32, device=dev)
            if with_sel and L.get("sel") is None:
                L["sel"] = torch.empty(2, dtype=torch.int32, device=dev)
                L["gates"] = torch.empty(2, dtype=torch.float32, device=dev)
        nbytes = wq.wq_moe_step_workspace_bytes(len(self.layers))
        self.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        layers = [(L["x"], L["logits"], L["w13"], L["s13"], L["w2"], L["s2"], L["work"], L.get("y32"), L["y16"],
                   L.get("sel"), L.get("gates")) for L in self.layers]
        self.plan = wq.wq_moe_step_prepare(self.e, self.dim, self.f, layers, self.workspace)
        return self.plan

    def step_fused(self, stream=None):
        """One decode step as two persistent launches (call prepare_fused first)."""
        wq.wq_moe_step_run(self.plan, stream)
