"""GPU parity of NF4 quantise/dequant and of the LoRA linear forward/backward
against the CPU oracle, on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth.configs import WORKLOADS
from tests.gpu_util import dev_bf16, dev, host, assert_close, oracle_weight

pytestmark = pytest.mark.gpu


def test_nf4_quantize_dequant_bitwise(gpu):
    w = synth.normal_bf16((192, 512), 0.02, 9, 0, 1)
    w[3, :64] = 0.0
    w[5, 64:128] = 0.0
    w[5, 100] = -0.375
    codes, absmax = gpu.nf4_quantize(dev_bf16(w))
    oc, oa = O.nf4_quantize(w.astype(np.float64))
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), oa.view(np.uint32))
    deq = gpu.nf4_dequant(codes, absmax)
    od = O.nf4_dequant(oc, oa)
    assert np.array_equal(host(deq), od)


def test_nf4_quantize_large_bitwise(gpu):
    # one Llama-8B-shaped o projection (4096 x 4096)
    w = synth.normal_bf16((4096, 4096), 0.02, 2, 0, 4)
    codes, absmax = gpu.nf4_quantize(dev_bf16(w))
    oc, oa = O.nf4_quantize(w.astype(np.float64))
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(absmax.cpu().numpy(), oa)


def test_nf4dq_absmax_quantize_dequant_bitwise(gpu):
    """Double quantization of the absmax on the GPU gives the oracle's bits: the
    8-bit codes, the per-256-block constants (a short last block, an all-zero
    block) and the dequantised weight."""
    from oracle.nf4 import nf4dq_quantize, nf4dq_dequant
    w = synth.normal_bf16((320, 448), 0.02, 12, 0, 1)     # 2240 absmax values: 8 full blocks + 192
    w[:37, :] = 0.0                                       # absmax block 0 all zero -> s = 0, q = 0
    w[40, 64:128] = 0.0                                   # a zero absmax inside a block
    codes, absmax = gpu.nf4_quantize(dev_bf16(w))
    q, scale = gpu.nf4dq_quantize_absmax(absmax)
    oc, oq, osc = nf4dq_quantize(w.astype(np.float64))
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert osc[0] == 0 and osc.size == 9
    deq = gpu.nf4dq_dequant(codes, q, scale)
    assert np.array_equal(host(deq), nf4dq_dequant(oc, oq, osc))


def test_nf4dq_absmax_rounding_ties(gpu):
    """absmax values that land exactly halfway between two 8-bit codes round to
    the even code on both sides (float32 division, then round-half-even)."""
    from oracle.nf4 import nf4dq_quantize_absmax
    s = np.float32(0.5) / np.float32(255.0)
    a = (np.arange(256, dtype=np.float32) + np.float32(0.5)) * s
    a[-1] = np.float32(0.5)                                # the block max -> code 255
    a = np.concatenate([a, np.float32([0.25, 0.0, 3e-3])]) # a short second block
    q, sc = gpu.nf4dq_quantize_absmax(dev(a))
    oq, osc = nf4dq_quantize_absmax(a)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32))


def _linear_case(T, fin, fout, r, alpha, wid, fmt, b_zero=False):
    x = synth.activation((T, fin), wid, "x")
    dy = synth.activation((T, fout), wid, "dy")
    w = synth.normal_bf16((fout, fin), 0.02, wid, 0, 1)
    a = synth.uniform_bf16((r, fin), -1 / np.sqrt(fin), 1 / np.sqrt(fin), wid, 0, 10)
    b = np.zeros((fout, r), np.float32) if b_zero else synth.normal_bf16((fout, r), 0.01, wid, 0, 11)
    return x, dy, w, a, b, alpha / r


@pytest.mark.parametrize("T,fin,fout,r,fmt", [
    (128, 256, 256, 8, "nf4"),        # single NF4 LoRA linear 256 -> 256, 128 tokens
    (200, 320, 448, 16, "nf4"),       # ragged: several tiles and a partial tile in T and both widths
    (200, 320, 448, 16, "bf16"),
    (1, 64, 64, 8, "nf4"),            # a single token, smallest shapes
    (200, 320, 448, 16, "nf4dq"),     # double-quantized absmax, short last 256-block
    (96, 1024, 1600, 8, "nf4dq"),
    # from 1024 tokens on, the GEMM tiles take 256 tokens:
    (1024, 512, 768, 16, "nf4"),      # whole token tiles
    (1300, 320, 448, 16, "nf4dq"),    # ragged tokens and weight rows
    (1024, 4096, 1024, 8, "nf4"),     # few output tiles: split-K, reduce in split order
    (300, 1024, 1152, 16, "bf16"),
    (128, 512, 256, 64, "bf16"),      # the largest rank of the linear API
    (64, 256, 384, 64, "nf4"),
    # at least 192 output tiles of 256 x 256: the large-tile GEMM. Forward:
    (1024, 256, 24576, 16, "nf4"),
    (1100, 320, 24576, 16, "bf16"),   # ragged tokens; bf16 weight tile by LDS DMA
    (1024, 256, 24640, 16, "nf4dq"),  # ragged weight rows (last tile 64 of 256)
    # input gradient ([K x N] weight layout):
    (1000, 24640, 192, 8, "nf4"),
    (1024, 24576, 256, 16, "bf16"),
    (1100, 24576, 320, 16, "nf4dq"),
    # large-tile pipeline edges: one and two K-steps, a single token
    (1024, 64, 24576, 8, "nf4"),
    (1100, 128, 24576, 16, "nf4dq"),
    (1024, 24576, 64, 8, "bf16"),
    (1, 64, 98304, 8, "nf4"),
    (1, 98304, 64, 8, "bf16"),
    # below 1024 tokens, fewer than 192 large tiles but at least 20 x 256 K-steps
    # in all: stream-K over 256 workgroups, split tiles summed by the last
    # arrival (the forward here; the input gradient has 192 tiles or more, one
    # per workgroup)
    (1000, 14336, 2048, 16, "nf4"),
    (900, 12288, 2048, 16, "nf4dq"),
    (1000, 2048, 14336, 8, "bf16"),   # the input gradient in stream-K, ragged tokens
    (900, 12288, 2112, 16, "nf4"),    # ragged weight rows (last tile 64 of 256), 27 steps per workgroup
    (512, 16384, 4096, 16, "bf16"),   # 32 steps per workgroup: forward tiles split exactly 8 ways;
                                      # input gradient two whole tiles per workgroup, nothing split
    # from 1024 tokens the same kind of shapes take large tiles with the
    # reduction split so that the splits fill the chip, partials summed in
    # split order by the reduce kernel
    (1024, 14336, 2048, 16, "nf4"),   # 32 tiles x 8 splits of 28 K-steps
    (1100, 12288, 2048, 16, "nf4dq"), # 40 tiles x 6 splits, ragged tokens
    (1024, 12288, 2112, 16, "nf4"),   # ragged weight rows, 36 tiles x 7 splits
    (1100, 4096, 4096, 16, "nf4dq"),  # 5 x 16 = 80 tiles, three splits of 22 K-steps, ragged tokens
    (1024, 2048, 4096, 16, "bf16"),   # forward 64 tiles x 4 splits, input gradient 32 tiles x 8 splits
])
def test_lora_linear_parity(gpu, T, fin, fout, r, fmt):
    x, dy, w, a, b, s = _linear_case(T, fin, fout, r, 2.0 * r, 1, fmt)
    if fmt in ("nf4", "nf4dq"):
        wd = oracle_weight(w, fmt)
        W = getattr(gpu.FrozenWeight, fmt)(dev_bf16(w))
    else:
        wd = w.astype(np.float64)
        W = gpu.FrozenWeight.dense(dev_bf16(w))
    xd, ad, bd, dyd = (v.astype(np.float64) for v in (x, a, b, dy))
    y_ref, t_ref = O.lora_linear_fwd(xd, wd, ad, bd, s)
    dx_ref, _, _, u_ref = O.lora_linear_bwd(xd, t_ref, dyd, wd, ad, bd, s)
    X, A, B, DY = dev_bf16(x), dev_bf16(a), dev_bf16(b), dev_bf16(dy)
    y, t = gpu.lora_linear_fwd(X, W, A, B, s)
    dA = torch.zeros((r, fin), dtype=torch.float32, device="cuda")
    dB = torch.zeros((fout, r), dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu.lora_linear_workspace_bytes(T, fout, fin, r), dtype=torch.uint8, device="cuda")
    dx = gpu.lora_linear_bwd(X, t, DY, W, A, B, s, dA, dB, ws=ws)
    u = gpu.lora_linear_bwd_u(ws, T, W, r).clone()
    torch.cuda.synchronize()
    assert_close(host(t), t_ref, "t")
    assert_close(host(u), u_ref, "u")
    assert_close(host(y), y_ref, "y")
    assert_close(host(dx), dx_ref, "dx")
    # the adapter gradients from the GPU's own bf16 t and u (a one-ulp rounding
    # difference in one of them moves a whole row of dA or dB)
    da_ref, db_ref = O.lora_adapter_grads(xd, host(t), dyd, host(u), s)
    assert_close(host(dA), da_ref, "dA")
    assert_close(host(dB), db_ref, "dB")
    # gradients accumulate (+=) in a fixed order: a second call doubles them exactly
    dA1, dB1 = dA.clone(), dB.clone()
    gpu.lora_linear_bwd(X, t, DY, W, A, B, s, dA, dB, need_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(dA, dA1 * 2) and torch.equal(dB, dB1 * 2)


@pytest.mark.parametrize("T,fin,fout,r,fmt", [
    (1000, 12288, 2112, 16, "nf4"),   # stream-K forward, split side products
    (300, 16384, 4096, 16, "bf16"),   # ragged tokens, stream-K both ways
    (1024, 4096, 4096, 16, "nf4"),    # the o projection's shape: large tiles, reduction split 4 ways
])
def test_split_partials_do_not_leak_between_calls(gpu, T, fin, fout, r, fmt):
    """Two calls with different inputs on one workspace: the second call's
    split partials land where the first call's still sit, and its results match
    the oracle for its own inputs (a partial read from the first call would
    not)."""
    ws_f = torch.empty(gpu.lora_linear_workspace_bytes(T, fout, fin, r), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty_like(ws_f)
    for wid in (5, 6):
        x, dy, w, a, b, s = _linear_case(T, fin, fout, r, 2.0 * r, wid, fmt)
        wd = oracle_weight(w, fmt)
        W = gpu.FrozenWeight.nf4(dev_bf16(w)) if fmt == "nf4" else gpu.FrozenWeight.dense(dev_bf16(w))
        xd, ad, bd, dyd = (v.astype(np.float64) for v in (x, a, b, dy))
        X, A, B, DY = dev_bf16(x), dev_bf16(a), dev_bf16(b), dev_bf16(dy)
        y, t = gpu.lora_linear_fwd(X, W, A, B, s, ws=ws_f)
        dA = torch.zeros((r, fin), dtype=torch.float32, device="cuda")
        dB = torch.zeros((fout, r), dtype=torch.float32, device="cuda")
        dx = gpu.lora_linear_bwd(X, t, DY, W, A, B, s, dA, dB, ws=ws_b)
        u = gpu.lora_linear_bwd_u(ws_b, T, W, r).clone()
        torch.cuda.synchronize()
        y_ref, t_ref = O.lora_linear_fwd(xd, wd, ad, bd, s)
        dx_ref, _, _, u_ref = O.lora_linear_bwd(xd, t_ref, dyd, wd, ad, bd, s)
        assert_close(host(t), t_ref, f"t, call {wid}")
        assert_close(host(y), y_ref, f"y, call {wid}")
        assert_close(host(u), u_ref, f"u, call {wid}")
        assert_close(host(dx), dx_ref, f"dx, call {wid}")
        da_ref, db_ref = O.lora_adapter_grads(xd, host(t), dyd, host(u), s)
        assert_close(host(dA), da_ref, f"dA, call {wid}")
        assert_close(host(dB), db_ref, f"dB, call {wid}")


@pytest.mark.parametrize("T,fin,fout,r,fmt", [
    (200, 320, 448, 16, "bf16"),      # ragged, unsplit GEMM
    (64, 4096, 512, 16, "nf4"),       # few output tiles: split-K path, bias added in the split reduce
    (1100, 256, 24576, 16, "nf4"),    # 256 x 256 tiles
    (1000, 14336, 2048, 16, "nf4"),   # stream-K: the bias added by the last arrival
    (1024, 14336, 2048, 16, "nf4"),   # large tiles, split reduction: the bias added in the reduce
])
def test_lora_linear_bias(gpu, T, fin, fout, r, fmt):
    """A frozen bias joins the forward sum before its single rounding; the
    backward ignores it."""
    x, dy, w, a, b, s = _linear_case(T, fin, fout, r, 2.0 * r, 4, fmt)
    bias = synth.normal_bf16((fout,), 0.5, 4, 0, 60)
    wd = oracle_weight(w, fmt)
    W0 = gpu.FrozenWeight.nf4(dev_bf16(w)) if fmt == "nf4" else gpu.FrozenWeight.dense(dev_bf16(w))
    W = W0.with_bias(dev_bf16(bias))
    xd, ad, bd = (v.astype(np.float64) for v in (x, a, b))
    y_ref, t_ref = O.lora_linear_fwd(xd, wd, ad, bd, s, bias=bias.astype(np.float64))
    X, A, B, DY = dev_bf16(x), dev_bf16(a), dev_bf16(b), dev_bf16(dy)
    y, t = gpu.lora_linear_fwd(X, W, A, B, s)
    y0, _ = gpu.lora_linear_fwd(X, W0, A, B, s)
    dA = torch.zeros((r, fin), dtype=torch.float32, device="cuda")
    dB = torch.zeros((fout, r), dtype=torch.float32, device="cuda")
    dA0, dB0 = dA.clone(), dB.clone()
    dx = gpu.lora_linear_bwd(X, t, DY, W, A, B, s, dA, dB)
    dx0 = gpu.lora_linear_bwd(X, t, DY, W0, A, B, s, dA0, dB0)
    torch.cuda.synchronize()
    assert_close(host(y), y_ref, "y with bias")
    assert not torch.equal(y, y0)
    assert torch.equal(dx, dx0) and torch.equal(dA, dA0) and torch.equal(dB, dB0)


def test_zero_b_is_plain_dequant_gemm(gpu):
    """B = 0 (LoRA init): y equals the product with the dequantised weight; the
    fused NF4 path and the dense path over the dequantised weight agree bitwise."""
    T, fin, fout, r = 256, 512, 384, 16
    x, dy, w, a, b, s = _linear_case(T, fin, fout, r, 32.0, 3, "nf4", b_zero=True)
    Wn = gpu.FrozenWeight.nf4(dev_bf16(w))
    Wd = gpu.FrozenWeight.dense(gpu.nf4_dequant(Wn.codes, Wn.absmax))
    X, A, B = dev_bf16(x), dev_bf16(a), dev_bf16(b)
    y1, _ = gpu.lora_linear_fwd(X, Wn, A, B, s)
    y2, _ = gpu.lora_linear_fwd(X, Wd, A, B, s)
    y3, _ = gpu.lora_linear_fwd(X, Wn, dev_bf16(a * 0.5), B, s)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    oc, oa = O.nf4_quantize(w.astype(np.float64))
    ref = O.round_bf16(x.astype(np.float64) @ O.nf4_dequant(oc, oa).T)
    assert_close(host(y1), ref, "y(B=0)")
    exact = np.mean(host(y1) == ref)
    print("fraction bitwise equal to the float64 product rounded once:", exact)
    assert exact > 0.95
