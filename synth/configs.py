"""Workload shapes (no arithmetic).

The shapes are those of the decoder-only bases the pages train (a Llama-3.1-8B
NF4 base and Qwen2.5 bf16 bases; "Exact Layer Streaming", abstract), with the
layer sizes of those public architectures. Small shapes exist so that the CPU
oracle finishes in seconds while still spanning several GPU tiles.
"""
from dataclasses import dataclass, field

# projection order used everywhere (tensor ids, LoRA parameter sets)
LORA_PROJ = ("q", "k", "v", "o", "gate", "up", "down")

# tensor ids inside one (workload, layer) stream family
TENSOR_IDS = {
    "norm1": 0, "q": 1, "k": 2, "v": 3, "o": 4, "norm2": 5,
    "gate": 6, "up": 7, "down": 8,
    # LoRA A / B per projection: 10 + 2*p and 11 + 2*p
    **{f"A_{p}": 10 + 2 * i for i, p in enumerate(LORA_PROJ)},
    **{f"B_{p}": 11 + 2 * i for i, p in enumerate(LORA_PROJ)},
    # activations
    "x": 40, "dy": 41, "tokens": 42,
    # model head (used with layer_id = HEAD_LAYER_ID)
    "embed": 50, "final_norm": 51, "lm_head": 52,
    # q/k/v bias (Qwen2 bases)
    "q_bias": 60, "k_bias": 61, "v_bias": 62,
}
HEAD_LAYER_ID = 1000


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    inter: int
    rms_eps: float
    rope_theta: float
    wfmt: str            # "nf4", "nf4dq" (double-quantized absmax) or "bf16"
    lora_r: int
    lora_alpha: float
    qkv_bias: bool = False          # Qwen2: frozen bias on q, k, v
    rope_scaling: tuple = None      # Llama-3.1: (factor, low_freq_factor, high_freq_factor, original_max_position)

    @property
    def lora_scale(self) -> float:
        return self.lora_alpha / self.lora_r

    @property
    def q_dim(self) -> int:
        return self.n_q * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv * self.head_dim


def PROJ_IN_OUT(s: LayerShape):
    """(in_features, out_features) of each projection, weights stored [out x in]."""
    return {
        "q": (s.hidden, s.q_dim), "k": (s.hidden, s.kv_dim), "v": (s.hidden, s.kv_dim),
        "o": (s.q_dim, s.hidden),
        "gate": (s.hidden, s.inter), "up": (s.hidden, s.inter),
        "down": (s.inter, s.hidden),
    }


@dataclass(frozen=True)
class ModelShape:
    layer: LayerShape
    n_layers: int
    vocab: int
    tied: bool            # lm_head shares the embedding table
    batch: int
    seq: int
    n_micro: int = 1
    adamw: bool = True


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int              # seed component
    kind: str             # "linear" | "layer" | "model"
    layer: LayerShape = None
    model: ModelShape = None
    tokens: int = 0       # linear / layer: T
    batch: int = 1
    seq: int = 0
    lin_in: int = 0
    lin_out: int = 0
    extra: dict = field(default_factory=dict)


LLAMA8B_LAYER = LayerShape(4096, 32, 8, 128, 14336, 1e-5, 500000.0, "nf4", 16, 32.0)
LLAMA8B_LAYER_DQ = LayerShape(4096, 32, 8, 128, 14336, 1e-5, 500000.0, "nf4dq", 16, 32.0)
QWEN05B_LAYER = LayerShape(896, 14, 2, 64, 4864, 1e-6, 1000000.0, "bf16", 16, 32.0)
QWEN3B_LAYER = LayerShape(2048, 16, 2, 128, 11008, 1e-6, 1000000.0, "bf16", 16, 32.0)

WORKLOADS = {
    # single NF4 LoRA linear 256 -> 256, 128 tokens, rank 8, alpha 16
    "linear_nf4_256": Workload("linear_nf4_256", 1, "linear", tokens=128,
                               lin_in=256, lin_out=256,
                               layer=LayerShape(256, 2, 2, 128, 256, 1e-5, 1e4, "nf4", 8, 16.0)),
    # one Llama-3.1-8B-shaped decoder layer, batch 1 x seq 512
    "llama8b_layer_s512": Workload("llama8b_layer_s512", 2, "layer", layer=LLAMA8B_LAYER,
                                   tokens=512, batch=1, seq=512),
    # Qwen2.5-0.5B-shaped model, bf16 base, 4 x 512 tokens, 4 microbatches
    "qwen05b_bf16": Workload("qwen05b_bf16", 3, "model", layer=QWEN05B_LAYER,
                             model=ModelShape(QWEN05B_LAYER, 24, 151936, True, 4, 512, 4)),
    # Qwen2.5-3B-shaped model, bf16 base, tied embeddings, 1 x 1024 tokens
    "qwen3b_bf16": Workload("qwen3b_bf16", 4, "model", layer=QWEN3B_LAYER,
                            model=ModelShape(QWEN3B_LAYER, 36, 151936, True, 1, 1024, 1)),
    # Llama-3.1-8B-shaped model, NF4 base, bf16 lm_head, 1 x 1024 tokens, AdamW step
    "llama8b_nf4": Workload("llama8b_nf4", 5, "model", layer=LLAMA8B_LAYER,
                            model=ModelShape(LLAMA8B_LAYER, 32, 128256, False, 1, 1024, 1)),
    # the same model with double-quantized absmax (the layer format of the pages' 4 GB runs)
    "llama8b_nf4dq": Workload("llama8b_nf4dq", 6, "model", layer=LLAMA8B_LAYER_DQ,
                              model=ModelShape(LLAMA8B_LAYER_DQ, 32, 128256, False, 1, 1024, 1)),
}

# the published Llama-3.1 RoPE frequency scaling (rope_type "llama3")
LLAMA31_ROPE_SCALING = (8.0, 1.0, 4.0, 8192.0)

# small shapes for the oracle's own checks and for quick GPU parity cases
TINY_LAYER = LayerShape(64, 4, 2, 16, 128, 1e-5, 10000.0, "nf4", 4, 8.0)
SMALL_LAYER_NF4 = LayerShape(256, 4, 2, 64, 512, 1e-5, 500000.0, "nf4", 16, 32.0)
SMALL_LAYER_BF16 = LayerShape(192, 3, 1, 64, 320, 1e-6, 1000000.0, "bf16", 8, 16.0)
SMALL_LAYER_NF4DQ = LayerShape(320, 5, 1, 64, 448, 1e-5, 500000.0, "nf4dq", 8, 16.0)
