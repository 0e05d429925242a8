"""The layer pool on the GPU: every state error of the slot life cycle and the
pinned-memory check reject the call before anything is enqueued; the poison
mode really fills a slot before its load; and streamed runs stay bit-identical
to resident ones with poisoned slots and with layers larger than the ~165 MiB
size above which the pages report silently wrong gradients ("Soup CLI ...",
"v0.73.0: Fixing Silent Wrong Gradients")."""
import ctypes as C
import dataclasses
import os

import numpy as np
import pytest
import torch

from layer_streamed_lora_amd import _abi
from layer_streamed_lora_amd.ops import lib
from synth.configs import LLAMA8B_LAYER

pytestmark = pytest.mark.gpu


def _pool(n_slots, slot_bytes):
    from layer_streamed_lora_amd.trainer import copy_stream
    slots = [torch.empty(slot_bytes, dtype=torch.uint8, device="cuda") for _ in range(n_slots)]
    ptrs = (C.c_void_p * n_slots)(*[s.data_ptr() for s in slots])
    h = C.c_void_p()
    assert lib().lsl_pool_create(C.byref(h), ptrs, n_slots, slot_bytes, copy_stream().cuda_stream) == _abi.LSL_OK
    return h, slots


def test_pool_state_and_pinning_errors(gpu):
    L = lib()
    nb = 1 << 16
    h, slots = _pool(2, nb)
    src = torch.arange(nb, dtype=torch.int32).to(torch.uint8).pin_memory()
    src2 = (torch.arange(nb, dtype=torch.int32) * 7).to(torch.uint8).pin_memory()
    got = C.c_void_p()
    try:
        # nothing loaded yet: acquire, release and reuse are out of order
        assert L.lsl_pool_acquire(h, 0, None, C.byref(got)) == _abi.LSL_ERR_STATE
        assert L.lsl_pool_release(h, 0, None) == _abi.LSL_ERR_STATE
        assert L.lsl_pool_reuse(h, 0) == _abi.LSL_ERR_STATE
        # pageable host memory, an oversized copy, a slot out of range
        pageable = np.zeros(nb, np.uint8)
        assert L.load_layer_async(h, 0, pageable.ctypes.data, nb) == _abi.LSL_ERR_NOT_PINNED
        assert L.load_layer_async(h, 0, src.data_ptr(), nb + 1) == _abi.LSL_ERR_INVALID_ARG
        assert L.load_layer_async(h, 2, src.data_ptr(), nb) == _abi.LSL_ERR_INVALID_ARG
        # loaded: a second load and a reuse are out of order
        assert L.load_layer_async(h, 0, src.data_ptr(), nb) == _abi.LSL_OK
        assert L.load_layer_async(h, 0, src2.data_ptr(), nb) == _abi.LSL_ERR_STATE
        assert L.lsl_pool_reuse(h, 0) == _abi.LSL_ERR_STATE
        assert L.lsl_pool_release(h, 0, None) == _abi.LSL_ERR_STATE
        # acquired: load, reuse and a second acquire are out of order
        assert L.lsl_pool_acquire(h, 0, None, C.byref(got)) == _abi.LSL_OK
        assert got.value == slots[0].data_ptr()
        assert L.load_layer_async(h, 0, src2.data_ptr(), nb) == _abi.LSL_ERR_STATE
        assert L.lsl_pool_reuse(h, 0) == _abi.LSL_ERR_STATE
        assert L.lsl_pool_acquire(h, 0, None, C.byref(got)) == _abi.LSL_ERR_STATE
        torch.cuda.synchronize()
        assert torch.equal(slots[0].cpu(), src)  # the rejected loads enqueued nothing
        # released: a second release is out of order; reuse and a new load are fine
        assert L.lsl_pool_release(h, 0, None) == _abi.LSL_OK
        assert L.lsl_pool_release(h, 0, None) == _abi.LSL_ERR_STATE
        assert L.lsl_pool_acquire(h, 0, None, C.byref(got)) == _abi.LSL_ERR_STATE
        assert L.lsl_pool_reuse(h, 0) == _abi.LSL_OK
        assert L.lsl_pool_acquire(h, 0, None, C.byref(got)) == _abi.LSL_OK
        assert L.lsl_pool_release(h, 0, None) == _abi.LSL_OK
        assert L.load_layer_async(h, 0, src2.data_ptr(), nb) == _abi.LSL_OK
        assert L.lsl_pool_acquire(h, 0, None, C.byref(got)) == _abi.LSL_OK
        torch.cuda.synchronize()
        assert torch.equal(slots[0].cpu(), src2)
        # the other slot was never touched
        assert L.lsl_pool_acquire(h, 1, None, C.byref(got)) == _abi.LSL_ERR_STATE
    finally:
        L.lsl_pool_destroy(h)


def test_poison_mode_fills_the_slot_before_each_load(gpu, monkeypatch):
    """With LSL_POISON_SLOTS the bytes of a slot past a short load read 0xFF
    (the fill ran on the copy stream, ahead of the copy); without it they keep
    what was there."""
    nb, part = 1 << 16, 1000
    src = torch.full((part,), 3, dtype=torch.uint8).pin_memory()
    for poison in (True, False):
        if poison:
            monkeypatch.setenv("LSL_POISON_SLOTS", "1")
        else:
            monkeypatch.delenv("LSL_POISON_SLOTS", raising=False)
        h, slots = _pool(1, nb)
        slots[0].fill_(5)
        torch.cuda.synchronize()
        try:
            assert lib().load_layer_async(h, 0, src.data_ptr(), part) == _abi.LSL_OK
            assert lib().lsl_pool_acquire(h, 0, None, None) == _abi.LSL_OK
            torch.cuda.synchronize()
            got = slots[0].cpu()
            assert torch.all(got[:part] == 3)
            assert torch.all(got[part:] == (255 if poison else 5))
        finally:
            lib().lsl_pool_destroy(h)


@pytest.mark.timeout(900)
def test_streamed_equals_resident_with_poisoned_slots(gpu, monkeypatch):
    """Streamed == resident, bit for bit, with every slot poisoned before each of
    its loads: a small NF4 model over two steps of three microbatches and the
    Llama-3.1-8B-shaped NF4 model (one step)."""
    from tests.test_gpu_model import _streamed_vs_resident, SMALL_NF4
    monkeypatch.setenv("LSL_POISON_SLOTS", "1")
    _streamed_vs_resident(SMALL_NF4, 5, 640, False, 2, 64, 3, 91)
    _streamed_vs_resident(LLAMA8B_LAYER, 32, 128256, False, 1, 1024, 1, 92)


@pytest.mark.timeout(900)
def test_streamed_equals_resident_layers_above_165mib(gpu, monkeypatch):
    """Three Llama-3.1-8B-shaped layers with an un-quantized bf16 base: each
    layer blob is 436 MB (416 MiB), far above the ~165 MiB per layer past which
    the pages' system produced wrong gradients; streamed (poisoned slots) and
    resident runs give identical bits over two microbatches."""
    from tests.test_gpu_model import _streamed_vs_resident
    monkeypatch.setenv("LSL_POISON_SLOTS", "1")
    shape = dataclasses.replace(LLAMA8B_LAYER, wfmt="bf16")
    s = _streamed_vs_resident(shape, 3, 32000, False, 1, 1024, 2, 93)
    assert s.blob_bytes > 165 * 2 ** 20 * 2
