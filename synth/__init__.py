"""Seeded synthetic inputs and workload shapes shared by the GPU path and the oracle.

This package holds data preparation only: shapes of the workloads and seeded
random tensors of the distributions the workloads use. It contains none of the
method's arithmetic (no quantisation, no matmul, no normalisation).

Every tensor is drawn from its own counter-free stream:
``numpy.random.Generator(PCG64(SeedSequence([workload_id, layer_id, tensor_id, salt])))``
so the oracle and the GPU harness see the same bytes whatever order they ask in.
Floating tensors are drawn in float32 and rounded to the nearest bfloat16
(ties to even), then returned as float32 arrays whose values are exactly
representable in bfloat16; ``as_bf16_bits`` gives the raw 16-bit patterns.
"""
from .configs import (  # noqa: F401
    LayerShape, ModelShape, WORKLOADS, TENSOR_IDS, LORA_PROJ, PROJ_IN_OUT,
)
from .gen import (  # noqa: F401
    stream, normal_bf16, uniform_bf16, norm_weight_bf16, token_ids,
    as_bf16_bits, layer_weights, layer_lora, model_head, activation,
)
