"""Whole training steps: the streamed model against the oracle (small shapes),
and streamed against resident bit for bit (the pages' correctness protocol:
"Exact Layer Streaming ...", abstract; "Soup CLI ...", section "How Layer
Streaming Works")."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth.configs import LayerShape, PROJ_IN_OUT, QWEN05B_LAYER, QWEN3B_LAYER, LLAMA8B_LAYER, LLAMA8B_LAYER_DQ
from tests.gpu_util import dev_bf16, host, assert_close_chain, oracle_layer_weights

pytestmark = pytest.mark.gpu

SMALL_NF4 = LayerShape(128, 2, 1, 64, 192, 1e-5, 500000.0, "nf4", 8, 16.0)
SMALL_BF16 = LayerShape(192, 3, 1, 64, 256, 1e-6, 1000000.0, "bf16", 16, 32.0)
SMALL_NF4DQ = LayerShape(192, 4, 1, 64, 320, 1e-5, 500000.0, "nf4dq", 16, 32.0)
# Qwen2-style q/k/v bias; Llama-3.1-style RoPE scaling with a short original context
SMALL_BF16_BIAS = LayerShape(192, 3, 1, 64, 256, 1e-6, 1000000.0, "bf16", 16, 32.0, qkv_bias=True)
SMALL_NF4_SCALED = LayerShape(128, 2, 1, 64, 192, 1e-5, 500000.0, "nf4", 8, 16.0,
                              rope_scaling=(8.0, 1.0, 4.0, 32.0))


def build(shape, n_layers, vocab, tied, batch, seq, mode, wid, keep_t=True):
    from layer_streamed_lora_amd.trainer import StreamedLoraModel
    m = StreamedLoraModel(shape, n_layers, vocab, tied, batch, seq, mode=mode, keep_t=keep_t)
    weights, loras = [], []
    for l in range(n_layers):
        w = synth.layer_weights(shape, wid, l, ones_norm=False)
        lo = synth.layer_lora(shape, wid, l)
        m.set_layer_weights(l, {k: dev_bf16(v) for k, v in w.items()})
        m.lora.set_from(l, lo)
        weights.append(w)
        loras.append(lo)
    emb, fn, lm = synth.model_head(shape.hidden, vocab, tied, wid, std=0.05, ones_norm=False)
    m.embed.copy_(dev_bf16(emb))
    m.final_norm.copy_(dev_bf16(fn))
    if not tied:
        m.lm_head.copy_(dev_bf16(lm))
    torch.cuda.synchronize()
    return m, weights, loras, (emb, fn, lm)


def ids_for(vocab, batch, seq, n_micro, wid):
    return [synth.token_ids(batch * seq, vocab, wid, salt=i) for i in range(n_micro)]


@pytest.mark.parametrize("shape,tied", [(SMALL_NF4, False), (SMALL_BF16, True), (SMALL_NF4DQ, False),
                                        (SMALL_BF16_BIAS, True), (SMALL_NF4_SCALED, False)])
def test_model_step_matches_oracle(gpu, shape, tied):
    n_layers, vocab, batch, seq, n_micro, wid = 3, 640, 2, 40, 2, 70
    m, weights, loras, (emb, fn, lm) = build(shape, n_layers, vocab, tied, batch, seq, "streamed", wid)
    chunks = ids_for(vocab, batch, seq, n_micro, wid)
    losses = m.step(m.prepare_inputs(chunks), adamw=False)
    torch.cuda.synchronize()
    layers = []
    for l in range(n_layers):
        wd = {}
        wd.update(oracle_layer_weights(weights[l], shape))
        wd["norm1"] = weights[l]["norm1"].astype(np.float64)
        wd["norm2"] = weights[l]["norm2"].astype(np.float64)
        layers.append((wd, {k: v.astype(np.float64) for k, v in loras[l].items()}))
    loss_ref, grads_ref, outs = O.model_step(chunks, emb.astype(np.float64), fn.astype(np.float64),
                                             None if tied else lm.astype(np.float64), layers, shape, batch, seq)
    got_losses = host(losses)
    for i in range(n_micro):
        assert abs(got_losses[i] - outs[i]["loss"]) <= 1e-3 * abs(outs[i]["loss"]), (got_losses[i], outs[i]["loss"])
    for l in range(n_layers):
        g = m.lora.grads_np(l)
        for k in grads_ref[l]:
            assert_close_chain(g[k], grads_ref[l][k], f"layer {l} {k}")


def _assert_same_state(a, b):
    for name in ("grad", "master", "bf16", "m", "v"):
        assert torch.equal(getattr(a.lora, name), getattr(b.lora, name)), name


@pytest.mark.parametrize("shape", [SMALL_NF4, SMALL_BF16, SMALL_NF4DQ, SMALL_BF16_BIAS])
def test_streamed_equals_resident_small(gpu, shape):
    n_layers, vocab, batch, seq, n_micro = 4, 640, 2, 64, 3
    s, *_ = build(shape, n_layers, vocab, False, batch, seq, "streamed", 71)
    r, *_ = build(shape, n_layers, vocab, False, batch, seq, "resident", 71)
    # the backward recomputing the LoRA products t instead of taking them from
    # the forward: the same bits
    n, *_ = build(shape, n_layers, vocab, False, batch, seq, "streamed", 71, keep_t=False)
    for step in range(2):
        chunks = ids_for(vocab, batch, seq, n_micro, 71 + step)
        ls = s.step(s.prepare_inputs(chunks))
        lr = r.step(r.prepare_inputs(chunks))
        ln = n.step(n.prepare_inputs(chunks))
        torch.cuda.synchronize()
        assert torch.equal(ls, lr) and torch.equal(ls, ln)
        assert torch.equal(s.ckpt, r.ckpt) and torch.equal(s.lse, r.lse)
        _assert_same_state(s, r)
        _assert_same_state(s, n)
    # every layer's adapters received gradient (no severed path)
    for l in range(n_layers):
        for i in range(4):
            assert torch.count_nonzero(s.lora.view(s.lora.grad, l, i, "A")) > 0
            assert torch.count_nonzero(s.lora.view(s.lora.grad, l, i, "B")) > 0
    # layer copies: 2L - 2 for the first microbatch, 2L - 4 for every later one
    # (the two layers at each turn of the sweep are reused from the slots)
    assert s.loads == (2 * n_layers - 2) + (2 * n_micro - 1) * (2 * n_layers - 4)


def _streamed_vs_resident(shape, L, V, tied, batch, seq, n_micro, seed):
    """Build a resident and a streamed model with the same random base
    (N(0, 0.02), unit norms), run one optimizer step on the same tokens and
    require identical bits everywhere."""
    from layer_streamed_lora_amd.trainer import StreamedLoraModel
    models = {}
    for mode in ("resident", "streamed"):
        m = StreamedLoraModel(shape, L, V, tied, batch, seq, mode=mode)
        g = torch.Generator(device="cuda").manual_seed(seed)
        for l in range(L):
            w = {}
            for p, (fin, fout) in PROJ_IN_OUT(shape).items():
                w[p] = (torch.randn((fout, fin), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
            w["norm1"] = torch.ones(shape.hidden, dtype=torch.bfloat16, device="cuda")
            w["norm2"] = torch.ones(shape.hidden, dtype=torch.bfloat16, device="cuda")
            if shape.qkv_bias:
                for p, n in (("q", shape.q_dim), ("k", shape.kv_dim), ("v", shape.kv_dim)):
                    w[p + "_bias"] = (torch.randn(n, generator=g, device="cuda") * 0.1).to(torch.bfloat16)
            m.set_layer_weights(l, w)
        m.embed.copy_((torch.randn((V, shape.hidden), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
        if not tied:
            m.lm_head.copy_((torch.randn((V, shape.hidden), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
        m.lora.master.copy_(torch.randn(m.lora.numel, generator=g, device="cuda") * 0.01)
        m.lora.bf16.copy_(m.lora.master.to(torch.bfloat16))
        models[mode] = m
    chunks = ids_for(V, batch, seq, n_micro, seed)
    out = {}
    for mode, m in models.items():
        out[mode] = m.step(m.prepare_inputs(chunks))
    torch.cuda.synchronize()
    s, r = models["streamed"], models["resident"]
    assert torch.equal(out["streamed"], out["resident"])
    assert torch.equal(s.ckpt, r.ckpt) and torch.equal(s.lse, r.lse)
    _assert_same_state(s, r)
    # one step: 2L - 2 copies for the first microbatch, 2L - 4 for each later one
    assert s.loads == (2 * L - 2) + (n_micro - 1) * (2 * L - 4)
    loss = host(out["streamed"]).mean()
    # random N(0, 0.02) weights: the loss sits near ln V
    assert abs(loss - np.log(V)) < 1.0, loss
    for l in (0, L - 1):
        assert torch.count_nonzero(s.lora.view(s.lora.grad, l, 0, "A")) > 0
    return s


@pytest.mark.timeout(900)
def test_streamed_equals_resident_qwen05b(gpu):
    """Qwen2.5-0.5B-shaped model (24 layers, hidden 896, 14/2 heads, MLP 4864,
    vocab 151936, tied), 4 microbatches of 4 x 512 tokens, one AdamW step:
    streamed and resident runs give identical bits."""
    _streamed_vs_resident(QWEN05B_LAYER, 24, 151936, True, 4, 512, 4, 3)


@pytest.mark.timeout(900)
def test_streamed_equals_resident_qwen3b(gpu):
    """Qwen2.5-3B-shaped model with an un-quantized bf16 base (36 layers,
    hidden 2048, 16/2 heads of 128, MLP 11008, vocab 151936, tied), 1 x 1024
    tokens: streamed (5.5 GB pinned store, two 154 MB slots) equals resident."""
    _streamed_vs_resident(QWEN3B_LAYER, 36, 151936, True, 1, 1024, 1, 4)


@pytest.mark.timeout(900)
def test_streamed_equals_resident_llama8b_nf4(gpu):
    """Llama-3.1-8B-shaped model, NF4 base (32 layers, 122.7 MB blobs, 3.9 GB
    pinned store), separate bf16 lm_head, vocab 128256, 1 x 1024 tokens."""
    _streamed_vs_resident(LLAMA8B_LAYER, 32, 128256, False, 1, 1024, 1, 5)


@pytest.mark.timeout(900)
def test_streamed_equals_resident_llama8b_nf4dq(gpu):
    """Llama-3.1-8B-shaped model with double-quantized absmax (112.5 MB layer
    blobs, 3.6 GB pinned store), 1 x 1024 tokens: streamed equals resident."""
    s = _streamed_vs_resident(LLAMA8B_LAYER_DQ, 32, 128256, False, 1, 1024, 1, 6)
    assert s.blob_bytes < 113_000_000


@pytest.mark.timeout(900)
def test_streamed_equals_resident_qwen05b_bias(gpu):
    """Qwen2.5-0.5B-shaped model as the real checkpoints are built: q/k/v bias
    (24 layers, tied head, 1 x 512 tokens, 2 microbatches)."""
    import dataclasses
    _streamed_vs_resident(dataclasses.replace(QWEN05B_LAYER, qkv_bias=True), 24, 151936, True, 1, 512, 2, 7)


@pytest.mark.timeout(900)
def test_streamed_equals_resident_llama8b_rope_scaled(gpu):
    """Llama-3.1-8B-shaped NF4 model with the published RoPE frequency scaling."""
    import dataclasses
    from synth.configs import LLAMA31_ROPE_SCALING
    _streamed_vs_resident(dataclasses.replace(LLAMA8B_LAYER, rope_scaling=LLAMA31_ROPE_SCALING), 32, 128256, False,
                          1, 1024, 1, 8)


@pytest.mark.parametrize("shape,tied", [(SMALL_NF4, False), (SMALL_BF16_BIAS, True)])
def test_reference_logprobs_match_oracle(gpu, shape, tied):
    """Adapter-off streamed forward + per-token log-probabilities against the
    oracle's reference forward (the adapters of the model are ignored)."""
    from oracle.model import reference_logprobs
    n_layers, vocab, batch, seq, n_micro, wid = 4, 640, 2, 40, 2, 72
    m, weights, loras, (emb, fn, lm) = build(shape, n_layers, vocab, tied, batch, seq, "streamed", wid)
    chunks = ids_for(vocab, batch, seq, n_micro, wid)
    loads0 = m.loads
    lp, slp = m.reference_logprobs(m.prepare_inputs(chunks))
    torch.cuda.synchronize()
    # every layer once per microbatch (a sweep ends holding layers L-2 and L-1, and the next starts at 0)
    assert m.loads - loads0 == n_micro * n_layers
    layer_w = []
    for l in range(n_layers):
        wd = {"norm1": weights[l]["norm1"].astype(np.float64), "norm2": weights[l]["norm2"].astype(np.float64)}
        wd.update(oracle_layer_weights(weights[l], shape))
        layer_w.append(wd)
    for i, ids in enumerate(chunks):
        ref, sref = reference_logprobs(ids, emb.astype(np.float64), fn.astype(np.float64),
                                       None if tied else lm.astype(np.float64), layer_w, shape, batch, seq)
        got = host(lp[i])
        # a chain of bf16 rounding points (every layer) precedes the scores: normwise and RMS-scaled bound
        assert_close_chain(got, ref, f"reference logp microbatch {i}")
        assert np.all(got.reshape(batch, seq)[:, -1] == 0)
        assert np.allclose(host(slp[i]), got.reshape(batch, seq).sum(1), rtol=1e-5)


def test_reference_logprobs_streamed_equals_resident_llama8b(gpu):
    """The adapter-off forward of the Llama-3.1-8B-shaped NF4 model, streamed
    (32 copies) and resident, gives identical bits; B = 0 adapters give the
    same scores through the training forward's loss."""
    import dataclasses
    s = _streamed_vs_resident(LLAMA8B_LAYER, 32, 128256, False, 1, 1024, 1, 5)
    from layer_streamed_lora_amd.trainer import StreamedLoraModel
    r = StreamedLoraModel(LLAMA8B_LAYER, 32, 128256, False, 1, 1024, mode="resident")
    r.copy_base_from(s)
    chunks = ids_for(128256, 1, 1024, 1, 9)
    loads0 = s.loads
    lps, slps = s.reference_logprobs(s.prepare_inputs(chunks))
    lpr, slpr = r.reference_logprobs(r.prepare_inputs(chunks))
    torch.cuda.synchronize()
    assert torch.equal(lps, lpr) and torch.equal(slps, slpr)
    # after the training step the slots hold layers 1 and 0, which the sweep reuses
    assert s.loads - loads0 == 32 - 2
    v = host(lps)[0, :-1]
    assert np.all(v < 0) and abs(-v.mean() - np.log(128256)) < 1.0


@pytest.mark.parametrize("n_layers,loads_first,loads_later", [
    (1, 1, 0),     # one layer: it never leaves its slot
    (2, 2, 0),     # two layers: both stay in the two slots
    (3, 4, 2),     # the turn reuses two of three
])
def test_streamed_equals_resident_few_layers(gpu, n_layers, loads_first, loads_later):
    """Models shorter than the two-slot sweep needs: streamed and resident runs
    give the same bits over two steps of two microbatches, with the copy counts
    that slot reuse implies, and one step matches the oracle."""
    shape, vocab, batch, seq, n_micro, wid = SMALL_NF4, 640, 2, 40, 2, 74
    s, weights, loras, (emb, fn, lm) = build(shape, n_layers, vocab, False, batch, seq, "streamed", wid)
    r, *_ = build(shape, n_layers, vocab, False, batch, seq, "resident", wid)
    chunks = ids_for(vocab, batch, seq, n_micro, wid)
    ls = s.step(s.prepare_inputs(chunks), adamw=False)
    lr = r.step(r.prepare_inputs(chunks), adamw=False)
    torch.cuda.synchronize()
    assert torch.equal(ls, lr)
    _assert_same_state(s, r)
    assert s.loads == loads_first + (n_micro - 1) * loads_later
    layers = []
    for l in range(n_layers):
        wd = {"norm1": weights[l]["norm1"].astype(np.float64), "norm2": weights[l]["norm2"].astype(np.float64)}
        wd.update(oracle_layer_weights(weights[l], shape))
        layers.append((wd, {k: v.astype(np.float64) for k, v in loras[l].items()}))
    _, grads_ref, outs = O.model_step(chunks, emb.astype(np.float64), fn.astype(np.float64), lm.astype(np.float64),
                                      layers, shape, batch, seq)
    for i in range(n_micro):
        assert abs(host(ls)[i] - outs[i]["loss"]) <= 1e-3 * abs(outs[i]["loss"])
    for l in range(n_layers):
        g = s.lora.grads_np(l)
        for k in grads_ref[l]:
            assert_close_chain(g[k], grads_ref[l][k], f"layer {l} {k}")
    # a second step (with AdamW) stays identical
    chunks2 = ids_for(vocab, batch, seq, n_micro, wid + 1)
    ls = s.step(s.prepare_inputs(chunks2))
    lr = r.step(r.prepare_inputs(chunks2))
    torch.cuda.synchronize()
    assert torch.equal(ls, lr)
    _assert_same_state(s, r)


def test_empty_inputs_are_no_ops(gpu):
    """Zero tokens: the layer, LoRA linear and cross-entropy calls succeed and
    write nothing (the loss of an empty batch is 0)."""
    from layer_streamed_lora_amd import model as M, _abi
    import ctypes as C
    from layer_streamed_lora_amd.ops import lib
    shape = SMALL_NF4
    cfg = M.layer_cfg(shape)
    L = M.layer_layout(cfg)
    blob = torch.zeros(L.total_bytes, dtype=torch.uint8, device="cuda")
    lp = M.LoraParams(shape, 1)
    sentinel = torch.full((8, shape.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for batch, seq in ((0, 16), (2, 0)):
        assert lib().decoder_layer_fwd(C.byref(cfg), blob.data_ptr(), C.byref(lp.lora_set(0)), sentinel.data_ptr(),
                                       batch, seq, sentinel.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                       None) == _abi.LSL_OK
        assert lib().decoder_layer_bwd(C.byref(cfg), blob.data_ptr(), C.byref(lp.lora_set(0)), sentinel.data_ptr(),
                                       sentinel.data_ptr(), batch, seq, sentinel.data_ptr(),
                                       C.byref(lp.lora_grads(0)), None, ws.data_ptr(), ws.numel(), None) == _abi.LSL_OK
    loss = torch.full((1,), 5.0, dtype=torch.float32, device="cuda")
    w = torch.zeros((64, shape.hidden), dtype=torch.bfloat16, device="cuda")
    assert lib().fused_ce_loss_fwd(None, w.data_ptr(), None, 0, shape.hidden, 64, -100, loss.data_ptr(), None,
                                   ws.data_ptr(), ws.numel(), None) == _abi.LSL_OK
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0) and loss.item() == 0.0
    assert torch.count_nonzero(lp.grad) == 0
