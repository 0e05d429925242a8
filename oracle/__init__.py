"""Plain CPU oracle for layer-streamed LoRA training.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never imports, calls or falls back to it, and this
package imports nothing from the product path.

What it computes is the plain definition of each step, in float64 numpy, with
an optional rounding function applied exactly where the GPU stores a bfloat16
tensor ("bf16 mode"); with ``rnd=identity`` ("exact mode") every function is the
exact mathematical map, which the tests differentiate by central finite
differences.

Sources (the pages are cited by title and section):
  * "Exact Layer Streaming: LoRA Fine-Tuning of an 8B Model on a 4 GB Laptop
    GPU", abstract: LoRA training of a frozen NF4 or bf16 base whose decoder
    layers are streamed; the streamed run must equal a resident run of the
    same numerics; the cross-entropy logits term; gradient accumulation.
  * "Soup CLI Lets You Fine-Tune an 8B LLM on a 4 GB Laptop GPU", section
    "How Layer Streaming Works": one decoder layer at a time, forward and
    backward; the base stays frozen.
  * NF4 itself is only named by the pages; its definition is the NormalFloat
    data type of QLoRA (Dettmers et al. 2023, section 3, "4-bit NormalFloat
    Quantization") with blockwise absmax scaling, block size 64.

Parity status: every function here is pinned by tests against closed forms,
library routines (torch CPU float64 ops, scipy), brute force or finite
differences; none is "parity unpinned". The model step (model.py: label
shift, embedding -> layers -> final norm -> head -> cross-entropy, and the
backward into every layer) is pinned against a torch float64 autograd
composition of library ops. The pages print no worked example of
the arithmetic; the one set of printed numbers that fixes a step is the byte
count of the double-quantized NF4 store (tests/golden/pages_store_sizes.json).
"""
from .bf16 import round_bf16, identity, bf16_bits, from_bf16_bits  # noqa: F401
from .nf4 import nf4_codebook, nf4_quantize, nf4_dequant  # noqa: F401
from .lora import lora_linear_fwd, lora_linear_bwd, lora_adapter_grads  # noqa: F401
from .layer import (  # noqa: F401
    rmsnorm_fwd, rmsnorm_bwd, rope_apply, rope_inv_freq, attention_fwd, attention_bwd,
    swiglu_fwd, swiglu_bwd, decoder_layer_fwd, decoder_layer_bwd,
)
from .ce import ce_loss_fwd, ce_loss_bwd  # noqa: F401
from .adamw import adamw_step  # noqa: F401
from .model import model_step  # noqa: F401
