"""GPU parity of the whole decoder layer (forward, and backward with recompute)
against the oracle, plus the determinism properties streaming relies on."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth.configs import SMALL_LAYER_NF4, SMALL_LAYER_BF16, SMALL_LAYER_NF4DQ, LLAMA8B_LAYER, PROJ_IN_OUT
from synth.configs import LLAMA31_ROPE_SCALING
from tests.gpu_util import dev_bf16, host, assert_close, assert_close_chain, oracle_layer_weights

pytestmark = pytest.mark.gpu


def _setup(gpu, shape, batch, seq, wid, ones_norm=False):
    from layer_streamed_lora_amd import model as M
    T = batch * seq
    w = synth.layer_weights(shape, wid, 0, ones_norm=ones_norm)
    lora = synth.layer_lora(shape, wid, 0)
    x = synth.activation((T, shape.hidden), wid, "x")
    dy = synth.activation((T, shape.hidden), wid, "dy")
    cfg = M.layer_cfg(shape)
    L = M.layer_layout(cfg)
    blob = torch.zeros(L.total_bytes, dtype=torch.uint8, device="cuda")
    M.write_layer_blob(shape, cfg, blob, {k: dev_bf16(v) for k, v in w.items()})
    lp = M.LoraParams(shape, 1)
    lp.set_from(0, lora)
    return M, cfg, blob, lp, w, lora, x, dy


def _oracle(shape, w, lora, x, dy, batch, seq):
    wd = {}
    wd.update(oracle_layer_weights(w, shape))
    wd["norm1"], wd["norm2"] = w["norm1"].astype(np.float64), w["norm2"].astype(np.float64)
    ld = {k: v.astype(np.float64) for k, v in lora.items()}
    xd, dyd = x.astype(np.float64), dy.astype(np.float64)
    out, _ = O.decoder_layer_fwd(xd, wd, ld, shape, batch, seq)
    dx, gr = O.decoder_layer_bwd(xd, dyd, wd, ld, shape, batch, seq)
    return out, dx, gr


def _run_and_compare(gpu, shape, batch, seq, wid):
    M, cfg, blob, lp, w, lora, x, dy = _setup(gpu, shape, batch, seq, wid)
    X, DY = dev_bf16(x), dev_bf16(dy)
    out = M.decoder_layer_fwd(cfg, blob, lp.lora_set(0), X, batch, seq)
    dx = M.decoder_layer_bwd(cfg, blob, lp.lora_set(0), X, DY, batch, seq, lp.lora_grads(0))
    torch.cuda.synchronize()
    out_ref, dx_ref, gr_ref = _oracle(shape, w, lora, x, dy, batch, seq)
    assert_close_chain(host(out), out_ref, "layer out")
    assert_close_chain(host(dx), dx_ref, "layer dx")
    got = lp.grads_np(0)
    for k in gr_ref:
        assert_close_chain(got[k], gr_ref[k], "grad " + k)
    return M, cfg, blob, lp, X, DY, out, dx


@pytest.mark.parametrize("shape,batch,seq", [
    (SMALL_LAYER_NF4, 2, 40),     # NF4, two sequences, partial tiles everywhere
    (SMALL_LAYER_BF16, 1, 150),   # bf16 base, group of 3, rank 8
    (SMALL_LAYER_NF4DQ, 1, 72),   # NF4 with double-quantized absmax, short last 256-block
    # Qwen2-style q/k/v bias with RoPE scaling past a 64-position original context
    (dataclasses.replace(SMALL_LAYER_BF16, qkv_bias=True, rope_scaling=(8.0, 1.0, 4.0, 64.0)), 1, 150),
    # NF4 with Llama-3.1's published RoPE scaling
    (dataclasses.replace(SMALL_LAYER_NF4, rope_scaling=LLAMA31_ROPE_SCALING), 2, 40),
    (SMALL_LAYER_NF4, 2, 600),    # 1200 tokens: 256-token GEMM tiles, one of them ragged
])
def test_layer_parity_small(gpu, shape, batch, seq):
    _run_and_compare(gpu, shape, batch, seq, 41)


@pytest.mark.timeout(900)
def test_layer_parity_llama8b_seq512(gpu):
    """One Llama-3.1-8B-shaped NF4 layer, batch 1 x seq 512, every output and gradient."""
    _run_and_compare(gpu, LLAMA8B_LAYER, 1, 512, 2)


def test_layer_large_tile_gemms_sampled_rows(gpu):
    """Llama-8B layer over 6144 one-token sequences: every projection GEMM, forward
    and input gradient, has at least 192 output tiles of 256 x 256 (the large-tile
    kernel, with the residual epilogues of o and down and the LoRA K-steps). With
    one token per sequence each output row depends on its own input row only, so
    the oracle checks sampled rows."""
    batch, seq = 6144, 1
    M, cfg, blob, lp, w, lora, x, dy = _setup(gpu, LLAMA8B_LAYER, batch, seq, 23)
    X, DY = dev_bf16(x), dev_bf16(dy)
    out = M.decoder_layer_fwd(cfg, blob, lp.lora_set(0), X, batch, seq)
    dx = M.decoder_layer_bwd(cfg, blob, lp.lora_set(0), X, DY, batch, seq, lp.lora_grads(0))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 1000, 2047, 3071, 4095, 4096, 5000, 6142, 6143])
    out_ref, dx_ref, _ = _oracle(LLAMA8B_LAYER, w, lora, x[rows], dy[rows], len(rows), 1)
    assert_close_chain(host(out)[rows], out_ref, "layer out (sampled rows)")
    assert_close_chain(host(dx)[rows], dx_ref, "layer dx (sampled rows)")


def test_layer_deterministic_and_address_independent(gpu):
    """Same bits from a second run and from a copy of the blob at another address
    (a streamed slot vs a resident copy)."""
    shape, batch, seq = SMALL_LAYER_NF4, 1, 96
    M, cfg, blob, lp, w, lora, x, dy = _setup(gpu, shape, batch, seq, 43)
    X, DY = dev_bf16(x), dev_bf16(dy)
    other = torch.empty(blob.numel() + 4096, dtype=torch.uint8, device="cuda")[1024:1024 + blob.numel()]
    other.copy_(blob)
    outs, dxs, grads = [], [], []
    for b in (blob, blob, other):
        lp.grad.zero_()
        outs.append(M.decoder_layer_fwd(cfg, b, lp.lora_set(0), X, batch, seq))
        dxs.append(M.decoder_layer_bwd(cfg, b, lp.lora_set(0), X, DY, batch, seq, lp.lora_grads(0)))
        grads.append(lp.grad.clone())
    torch.cuda.synchronize()
    for i in (1, 2):
        assert torch.equal(outs[0], outs[i]) and torch.equal(dxs[0], dxs[i]) and torch.equal(grads[0], grads[i])


@pytest.mark.parametrize("shape,batch,seq", [(SMALL_LAYER_NF4, 2, 40), (LLAMA8B_LAYER, 1, 1024)])
def test_layer_kept_t_gives_the_same_bits(gpu, shape, batch, seq):
    """A backward whose recompute takes the LoRA products t kept by the forward
    (t_keep) gives the same bits as one that computes them again: dx, every
    adapter gradient, and the kept t equal the workspace's recomputed t."""
    from layer_streamed_lora_amd import _abi
    M, cfg, blob, lp, w, lora, x, dy = _setup(gpu, shape, batch, seq, 47)
    X, DY = dev_bf16(x), dev_bf16(dy)
    tk = torch.full((M.layer_tkeep_bytes(cfg, batch, seq),), 0xFF, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(M.layer_workspace_bytes(cfg, batch, seq, _abi.MODE_BWD), dtype=torch.uint8, device="cuda")
    out0 = M.decoder_layer_fwd(cfg, blob, lp.lora_set(0), X, batch, seq)
    out1 = M.decoder_layer_fwd(cfg, blob, lp.lora_set(0), X, batch, seq, t_keep=tk)
    res = []
    for keep in (None, tk):
        lp.grad.zero_()
        dx = M.decoder_layer_bwd(cfg, blob, lp.lora_set(0), X, DY, batch, seq, lp.lora_grads(0), ws=wsb, t_keep=keep)
        res.append((dx, lp.grad.clone()))
        if keep is None:  # the recomputed t of this workspace, to compare with the kept ones
            m = M.layer_workspace_map(cfg, batch, seq, _abi.MODE_BWD)
            T, r = batch * seq, shape.lora_r
            t_ws = [wsb[m[n]:m[n] + T * k * r * 2].clone() for n, k in (("t_qkv", 3), ("t_o", 1), ("t_gu", 2),
                                                                          ("t_down", 1))]
    torch.cuda.synchronize()
    assert torch.equal(out0, out1)
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    off = 0
    for t, k in zip(t_ws, (3, 1, 2, 1)):
        assert torch.equal(tk[off:off + t.numel()], t)
        off += (t.numel() + 255) // 256 * 256
    assert off == tk.numel()


@pytest.mark.parametrize("shape,seq", [
    (LLAMA8B_LAYER, 1024),
    (dataclasses.replace(LLAMA8B_LAYER, qkv_bias=True, rope_scaling=LLAMA31_ROPE_SCALING), 1024),
    (LLAMA8B_LAYER, 1100),  # a ragged last token tile
])
def test_layer_split_sums_fused_into_norms_give_the_standalone_bits(gpu, shape, seq):
    """At 1024 tokens the q|k|v and o projections and the gate|up and q|k|v input
    gradients of the Llama-8B layer leave split partials that the RoPE or
    RMSNorm after them sums: what those write must be the standalone RoPE and
    RMSNorm ops' bits on the bf16 tensors they write beside them (qkv -> the
    rotated q and k; h1 -> n2; dn2 -> dh1; dn1 -> dx)."""
    from layer_streamed_lora_amd import _abi
    batch = 1
    M, cfg, blob, lp, w, lora, x, dy = _setup(gpu, shape, batch, seq, 48, ones_norm=False)
    X, DY = dev_bf16(x), dev_bf16(dy)
    T, H, eps = batch * seq, shape.hidden, shape.rms_eps
    n1w, n2w = dev_bf16(w["norm1"]), dev_bf16(w["norm2"])
    wsf = torch.empty(M.layer_workspace_bytes(cfg, batch, seq, _abi.MODE_FWD), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(M.layer_workspace_bytes(cfg, batch, seq, _abi.MODE_BWD), dtype=torch.uint8, device="cuda")

    def region(ws, off):
        return ws[off:off + T * H * 2].view(torch.bfloat16).view(T, H)
    M.decoder_layer_fwd(cfg, blob, lp.lora_set(0), X, batch, seq, ws=wsf)
    mf = M.layer_workspace_map(cfg, batch, seq, _abi.MODE_FWD)
    h1, n2 = region(wsf, mf["h1"]).clone(), region(wsf, mf["n2"]).clone()
    sh = shape
    nqkv = (sh.n_q + 2 * sh.n_kv) * sh.head_dim
    qkv = wsf[mf["qkv"]:mf["qkv"] + T * nqkv * 2].view(torch.bfloat16).view(T, nqkv).clone()
    qkr = wsf[mf["qk_rope"]:mf["qk_rope"] + T * nqkv * 2].view(torch.bfloat16).view(T, nqkv).clone()
    nrot = (sh.n_q + sh.n_kv) * sh.head_dim
    rot = gpu.rope(qkv.clone(), sh.n_q + sh.n_kv, sh.head_dim, seq, sh.rope_theta, scaling=sh.rope_scaling)
    dx = M.decoder_layer_bwd(cfg, blob, lp.lora_set(0), X, DY, batch, seq, lp.lora_grads(0), ws=wsb)
    mb = M.layer_workspace_map(cfg, batch, seq, _abi.MODE_BWD)
    dn2, dh1, dn1 = (region(wsb, mb[k]).clone() for k in ("d_n2", "d_h1", "d_n1"))
    torch.cuda.synchronize()
    assert torch.equal(rot[:, :nrot], qkr[:, :nrot])
    assert torch.equal(gpu.rmsnorm_fwd(h1, n2w, eps), n2)
    assert torch.equal(gpu.rmsnorm_bwd(h1, n2w, dn2, eps, dres=DY), dh1)
    assert torch.equal(gpu.rmsnorm_bwd(X, n1w, dn1, eps, dres=dh1), dx)
    # the recomputed forward inside the backward wrote the same h1 and n2
    assert torch.equal(region(wsb, mb["h1"]), h1) and torch.equal(region(wsb, mb["n2"]), n2)


def test_layer_zero_b_gives_zero_dA(gpu):
    shape, batch, seq = SMALL_LAYER_BF16, 1, 64
    M, cfg, blob, lp, w, lora, x, dy = _setup(gpu, shape, batch, seq, 44)
    for i in range(4):
        lp.view(lp.bf16, 0, i, "B").zero_()
    M.decoder_layer_bwd(cfg, blob, lp.lora_set(0), dev_bf16(x), dev_bf16(dy), batch, seq, lp.lora_grads(0))
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.count_nonzero(lp.view(lp.grad, 0, i, "A")) == 0
        assert torch.count_nonzero(lp.view(lp.grad, 0, i, "B")) > 0


def test_layer_adapters_off(gpu):
    """lora = NULL runs the frozen base alone: the oracle's adapter-off layer,
    and bit for bit the GPU layer with every B = 0."""
    from layer_streamed_lora_amd import model as M
    shape, batch, seq = dataclasses.replace(SMALL_LAYER_BF16, qkv_bias=True), 2, 72
    M_, cfg, blob, lp, w, lora, x, dy = _setup(gpu, shape, batch, seq, 45)
    X = dev_bf16(x)
    off = M.decoder_layer_fwd(cfg, blob, None, X, batch, seq)
    lp0 = M.LoraParams(shape, 1)
    lp0.set_from(0, {k: (np.zeros_like(v) if k.startswith("B_") else v) for k, v in lora.items()})
    zero_b = M.decoder_layer_fwd(cfg, blob, lp0.lora_set(0), X, batch, seq)
    torch.cuda.synchronize()
    assert torch.equal(off, zero_b)
    wd = {"norm1": w["norm1"].astype(np.float64), "norm2": w["norm2"].astype(np.float64)}
    wd.update(oracle_layer_weights(w, shape))
    ref, _ = O.decoder_layer_fwd(x.astype(np.float64), wd, None, shape, batch, seq)
    assert_close_chain(host(off), ref, "adapter-off layer out")
