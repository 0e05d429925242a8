"""The allocation-free LoRA forward (lora_linear_fwd_noalloc, for callers that
cannot allocate device memory) against the workspace entry point
lora_linear_fwd through the C ABI: identical bits on two calls in a row, the
second with a smaller input, and a clear WORKSPACE error past its scratch."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def _case(gpu, T, n_out, k_in, r, wid, fmt):
    x = dev_bf16(synth.activation((T, k_in), wid, "x"))
    w = dev_bf16(synth.normal_bf16((n_out, k_in), 0.02, wid, 0, 1))
    W = gpu.FrozenWeight.nf4(w) if fmt == "nf4" else gpu.FrozenWeight.dense(w)
    A = dev_bf16(synth.uniform_bf16((r, k_in), -k_in ** -0.5, k_in ** -0.5, wid, 0, 10))
    B = dev_bf16(synth.normal_bf16((n_out, r), 0.01, wid, 0, 11))
    return x, W, A, B


def test_noalloc_forward_matches_workspace_forward(gpu):
    assert gpu.noalloc_scratch_bytes() == (88 << 20) + (64 << 10)
    # first the Llama-8B q|k|v projection at 1000 tokens, whose stream-K
    # partials fill 87.75 MiB of it; then a smaller, ragged call of the same
    # shape in bf16 (the array keeps the first call's partials and leaves its
    # arrival counts at zero; neither may leak into the second call)
    cases = [(1000, 6144, 4096, 16, "nf4"), (300, 6144, 4096, 16, "bf16")]
    assert gpu.lora_linear_workspace_bytes(1000, 6144, 4096, 16) >= 87 << 20
    for i, (T, n_out, k_in, r, fmt) in enumerate(cases):
        x, W, A, B = _case(gpu, T, n_out, k_in, r, 30 + i, fmt)
        y0, t0 = gpu.lora_linear_fwd(x, W, A, B, 2.0)
        y1 = torch.full((T, n_out), 7.0, dtype=torch.bfloat16, device="cuda")
        t1 = torch.full((T, r), 7.0, dtype=torch.bfloat16, device="cuda")
        gpu.lora_linear_fwd_noalloc(x, W, A, B, 2.0, y=y1, t=t1)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(t0, t1), (T, n_out, k_in)
        assert torch.count_nonzero(y1) > 0


def test_noalloc_forward_rejects_shapes_past_its_scratch(gpu):
    """1536 tokens of a 6144 x 4096 projection (144 large tiles) need 399
    stream-K slots of 256 KiB, more than the array holds; nothing is written."""
    from layer_streamed_lora_amd import _abi
    T, n_out, k_in, r = 1536, 6144, 4096, 16
    x, W, A, B = _case(gpu, T, n_out, k_in, r, 40, "nf4")
    y = torch.full((T, n_out), 7.0, dtype=torch.bfloat16, device="cuda")
    t = torch.full((T, r), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.LslError) as e:
        gpu.lora_linear_fwd_noalloc(x, W, A, B, 2.0, y=y, t=t)
    assert e.value.status == _abi.LSL_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and torch.all(t == 7.0)
