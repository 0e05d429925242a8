"""Every rounding point of the decoder layer, checked on its own.

After decoder_layer_fwd and decoder_layer_bwd each intermediate is read back
from the workspace (lsl_layer_workspace_map) and compared with the oracle step
that produces it, fed the GPU's own preceding tensors (teacher forcing), so no
error is carried from one step to the next. Each comparison holds the stated
bound |gpu - oracle| <= 1e-2 + 2e-2 |oracle| per element, with the absolute
term scaled down for tensors whose RMS is below 1 (tests/gpu_util.py,
assert_close_scaled); float32 adapter gradients and the attention statistics
are held to the same bound or tighter. Two outputs pass two rounding points
each because the first one is not stored (h1 = bf16(x + bf16(o projection))
and the layer output likewise); there the oracle rounds at both points too, and
the bound adds 2e-2 times the first sum's magnitude, the scale of its rounding
error (where x and the projection cancel, the output is far smaller).
The Llama-3.1-8B layer runs at seq 512
and at 1024 tokens, the dispatch the benchmark times (q|k|v and down forward and
the q|k|v and gate|up input gradients in stream-K large tiles, the o projection
both ways in large tiles with a split reduction, the gate|up forward and the
down input gradient one large tile per workgroup)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth.configs import SMALL_LAYER_NF4, SMALL_LAYER_BF16, SMALL_LAYER_NF4DQ, LLAMA8B_LAYER, LLAMA31_ROPE_SCALING
from tests.gpu_util import dev_bf16, host, assert_close_scaled, oracle_layer_weights

pytestmark = pytest.mark.gpu


def _region(ws, off, rows, cols, dtype=torch.bfloat16, use=None):
    """[rows x cols] at byte offset off; use: the first `use` columns only (the
    rest of the rows is never written and may hold any bits)."""
    n = rows * cols * (2 if dtype == torch.bfloat16 else 4)
    t = ws[off:off + n].view(dtype).view(rows, cols)
    return host(t if use is None else t[:, :use])


def _run(shape, batch, seq, wid):
    from layer_streamed_lora_amd import model as M
    from layer_streamed_lora_amd import _abi
    T = batch * seq
    w = synth.layer_weights(shape, wid, 0, ones_norm=False)
    lora = synth.layer_lora(shape, wid, 0)
    x = synth.activation((T, shape.hidden), wid, "x")
    dy = synth.activation((T, shape.hidden), wid, "dy")
    cfg = M.layer_cfg(shape)
    blob = torch.zeros(M.layer_layout(cfg).total_bytes, dtype=torch.uint8, device="cuda")
    M.write_layer_blob(shape, cfg, blob, {k: dev_bf16(v) for k, v in w.items()})
    lp = M.LoraParams(shape, 1)
    lp.set_from(0, lora)
    lp.grad.zero_()
    X, DY = dev_bf16(x), dev_bf16(dy)
    wsf = torch.empty(M.layer_workspace_bytes(cfg, batch, seq, _abi.MODE_FWD), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(M.layer_workspace_bytes(cfg, batch, seq, _abi.MODE_BWD), dtype=torch.uint8, device="cuda")
    out = M.decoder_layer_fwd(cfg, blob, lp.lora_set(0), X, batch, seq, ws=wsf)
    dx = M.decoder_layer_bwd(cfg, blob, lp.lora_set(0), X, DY, batch, seq, lp.lora_grads(0), ws=wsb)
    torch.cuda.synchronize()
    mf = M.layer_workspace_map(cfg, batch, seq, _abi.MODE_FWD)
    mb = M.layer_workspace_map(cfg, batch, seq, _abi.MODE_BWD)
    wd = oracle_layer_weights(w, shape)
    wd["norm1"], wd["norm2"] = w["norm1"].astype(np.float64), w["norm2"].astype(np.float64)
    ld = {k: v.astype(np.float64) for k, v in lora.items()}
    return dict(x=x.astype(np.float64), dy=dy.astype(np.float64), out=host(out), dx=host(dx), wsf=wsf, wsb=wsb,
                mf=mf, mb=mb, wd=wd, ld=ld, grads=lp.grads_np(0))


def _check_steps(shape, batch, seq, wid):
    r = _run(shape, batch, seq, wid)
    T, H, I, rk = batch * seq, shape.hidden, shape.inter, shape.lora_r
    Q, KV, d, nq, nkv = shape.q_dim, shape.kv_dim, shape.head_dim, shape.n_q, shape.n_kv
    NQKV = Q + 2 * KV
    s, eps, theta = shape.lora_scale, shape.rms_eps, shape.rope_theta
    sc = shape.rope_scaling
    pos = O.layer.positions_of(batch, seq)
    wd, ld, x, dy = r["wd"], r["ld"], r["x"], r["dy"]
    rnd = O.round_bf16
    wsb, mb = r["wsb"], r["mb"]

    def g(name, cols, rows=T, dtype=torch.bfloat16, use=None):
        return _region(wsb, mb[name], rows, cols, dtype, use)

    # the recompute in the backward equals the forward call bit for bit
    for name, cols in (("n1", H), ("qkv", NQKV), ("attn", Q), ("h1", H), ("gu", 2 * I), ("act", I)):
        assert np.array_equal(_region(r["wsf"], r["mf"][name], T, cols), g(name, cols)), name

    # ---- forward
    n1 = g("n1", H)
    assert_close_scaled(n1, O.rmsnorm_fwd(x, wd["norm1"], eps), "n1")
    ys, ts = [], []
    for p in ("q", "k", "v"):
        y, t = O.lora_linear_fwd(n1, wd[p], ld["A_" + p], ld["B_" + p], s, bias=wd.get(p + "_bias"))
        ys.append(y)
        ts.append(t)
    assert_close_scaled(g("t_qkv", 3 * rk), np.concatenate(ts, 1), "t_qkv")
    qkv = g("qkv", NQKV)
    assert_close_scaled(qkv, np.concatenate(ys, 1), "qkv")
    qkr = g("qk_rope", NQKV, use=Q + KV)
    qr_ref = O.rope_apply(qkv[:, :Q].reshape(T, nq, d), pos, theta, scaling=sc).reshape(T, Q)
    kr_ref = O.rope_apply(qkv[:, Q:Q + KV].reshape(T, nkv, d), pos, theta, scaling=sc).reshape(T, KV)
    assert_close_scaled(qkr, np.concatenate([qr_ref, kr_ref], 1), "q, k after RoPE")
    qr, kr, v = qkr[:, :Q].reshape(T, nq, d), qkr[:, Q:].reshape(T, nkv, d), qkv[:, Q + KV:].reshape(T, nkv, d)
    o_ref, lse_ref = O.attention_fwd(qr, kr, v, batch, seq)
    attn = g("attn", Q)
    assert_close_scaled(attn, o_ref.reshape(T, Q), "attention output")
    o_exact, _ = O.attention_fwd(qr, kr, v, batch, seq, rnd=O.identity)
    assert_close_scaled(g("attn32", Q, dtype=torch.float32), o_exact.reshape(T, Q), "attention output (float32)")
    lse = _region(wsb, mb["lse"], batch * nq, seq, torch.float32).reshape(batch, nq, seq)
    assert np.max(np.abs(lse - lse_ref) / (1.0 + np.abs(lse_ref))) <= 1e-5, "attention lse"
    y_o, t_o = O.lora_linear_fwd(attn, wd["o"], ld["A_o"], ld["B_o"], s)
    assert_close_scaled(g("t_o", rk), t_o, "t_o")
    h1 = g("h1", H)
    assert_close_scaled(h1, rnd(x + y_o), "h1 = x + o projection", inter=y_o)
    n2 = g("n2", H)
    assert_close_scaled(n2, O.rmsnorm_fwd(h1, wd["norm2"], eps), "n2")
    yg, tg = O.lora_linear_fwd(n2, wd["gate"], ld["A_gate"], ld["B_gate"], s)
    yu, tu = O.lora_linear_fwd(n2, wd["up"], ld["A_up"], ld["B_up"], s)
    assert_close_scaled(g("t_gu", 2 * rk), np.concatenate([tg, tu], 1), "t_gu")
    gu = g("gu", 2 * I)
    assert_close_scaled(gu, np.concatenate([yg, yu], 1), "gate|up")
    act = g("act", I)
    assert_close_scaled(act, O.swiglu_fwd(gu[:, :I], gu[:, I:]), "swiglu")
    y_d, t_d = O.lora_linear_fwd(act, wd["down"], ld["A_down"], ld["B_down"], s)
    assert_close_scaled(g("t_down", rk), t_d, "t_down")
    assert_close_scaled(r["out"], rnd(h1 + y_d), "layer output = h1 + down projection", inter=y_d)

    # ---- backward (and the float32 adapter gradients of each projection)
    grads = r["grads"]

    from oracle.lora import lora_adapter_grads

    def lin_bwd(xin, t_in, dout, p, u_gpu):
        """dx (unrounded) and u of one projection from the GPU's inputs; its
        adapter gradients from the GPU's own u (a one-ulp flip of u moves dA by
        more than the bound where dA cancels to about zero)."""
        dxp, _, _, u = O.lora_linear_bwd(xin, t_in, dout, wd[p], ld["A_" + p], ld["B_" + p], s, round_dx=False)
        dA, dB = lora_adapter_grads(xin, t_in, dout, u_gpu, s)
        assert_close_scaled(grads["A_" + p], dA, "dA_" + p)
        assert_close_scaled(grads["B_" + p], dB, "dB_" + p)
        return dxp, u

    u_down = g("u_down", rk)
    dxp, u = lin_bwd(act, g("t_down", rk), dy, "down", u_down)
    assert_close_scaled(u_down, u, "u_down")
    d_act = g("d_act", I)
    assert_close_scaled(d_act, rnd(dxp), "d_act")
    dg_ref, du_ref = O.swiglu_bwd(gu[:, :I], gu[:, I:], d_act)
    d_gu = g("d_gu", 2 * I)
    assert_close_scaled(d_gu, np.concatenate([dg_ref, du_ref], 1), "d_gate|d_up")
    t_gu, u_gu = g("t_gu", 2 * rk), g("u_gu", 2 * rk)
    dxg, ug = lin_bwd(n2, t_gu[:, :rk], d_gu[:, :I], "gate", u_gu[:, :rk])
    dxu, uu = lin_bwd(n2, t_gu[:, rk:], d_gu[:, I:], "up", u_gu[:, rk:])
    assert_close_scaled(u_gu, np.concatenate([ug, uu], 1), "u_gu")
    d_n2 = g("d_n2", H)
    assert_close_scaled(d_n2, rnd(dxg + dxu), "d_n2")
    d_h1 = g("d_h1", H)
    assert_close_scaled(d_h1, rnd(dy + O.rmsnorm_bwd(h1, wd["norm2"], eps, d_n2)), "d_h1")
    u_o = g("u_o", rk)
    dxo, uo = lin_bwd(attn, g("t_o", rk), d_h1, "o", u_o)
    assert_close_scaled(u_o, uo, "u_o")
    d_attn = g("d_attn", Q)
    assert_close_scaled(d_attn, rnd(dxo), "d_attn")
    dqr, dkr, dv = O.attention_bwd(qr, kr, v, d_attn.reshape(T, nq, d), batch, seq)
    dqkr = g("d_qk_rope", NQKV, use=Q + KV)
    assert_close_scaled(dqkr[:, :Q], dqr.reshape(T, Q), "dq (before inverse RoPE)")
    assert_close_scaled(dqkr[:, Q:Q + KV], dkr.reshape(T, KV), "dk (before inverse RoPE)")
    d_qkv = g("d_qkv", NQKV)
    assert_close_scaled(d_qkv[:, Q + KV:], dv.reshape(T, KV), "dv")
    dq_ref = O.rope_apply(dqkr[:, :Q].reshape(T, nq, d), pos, theta, inverse=True, scaling=sc).reshape(T, Q)
    dk_ref = O.rope_apply(dqkr[:, Q:Q + KV].reshape(T, nkv, d), pos, theta, inverse=True, scaling=sc).reshape(T, KV)
    assert_close_scaled(d_qkv[:, :Q + KV], np.concatenate([dq_ref, dk_ref], 1), "dq, dk (inverse RoPE)")
    t_qkv, u_qkv = g("t_qkv", 3 * rk), g("u_qkv", 3 * rk)
    dn1, us = 0.0, []
    for j, (p, c0, c1) in enumerate((("q", 0, Q), ("k", Q, Q + KV), ("v", Q + KV, NQKV))):
        dxp, u = lin_bwd(n1, t_qkv[:, j * rk:(j + 1) * rk], d_qkv[:, c0:c1], p, u_qkv[:, j * rk:(j + 1) * rk])
        dn1 = dn1 + dxp
        us.append(u)
    assert_close_scaled(u_qkv, np.concatenate(us, 1), "u_qkv")
    d_n1 = g("d_n1", H)
    assert_close_scaled(d_n1, rnd(dn1), "d_n1")
    assert_close_scaled(r["dx"], rnd(d_h1 + O.rmsnorm_bwd(x, wd["norm1"], eps, d_n1)), "dx")


@pytest.mark.parametrize("shape,batch,seq", [
    (SMALL_LAYER_NF4, 2, 40),
    (SMALL_LAYER_BF16, 1, 150),
    (SMALL_LAYER_NF4DQ, 1, 72),
    (dataclasses.replace(SMALL_LAYER_BF16, qkv_bias=True, rope_scaling=(8.0, 1.0, 4.0, 64.0)), 1, 150),
    (SMALL_LAYER_NF4, 2, 600),
])
def test_layer_steps_small(gpu, shape, batch, seq):
    _check_steps(shape, batch, seq, 81)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("shape,seq", [
    (LLAMA8B_LAYER, 512),
    (LLAMA8B_LAYER, 1024),
    # the split q|k|v sum inside the RoPE launch, with a q|k|v bias and
    # Llama-3.1's RoPE frequency scaling
    (dataclasses.replace(LLAMA8B_LAYER, qkv_bias=True, rope_scaling=LLAMA31_ROPE_SCALING), 1024),
    # a ragged last token tile (1100 = 4 x 256 + 76) in the split large tiles and
    # the RoPE / RMSNorm launches that sum their partials
    (LLAMA8B_LAYER, 1100),
])
def test_layer_steps_llama8b(gpu, shape, seq):
    """The Llama-3.1-8B NF4 layer at batch 1 x seq 512 and x 1024 (the
    benchmark's dispatch), every rounding point."""
    _check_steps(shape, 1, seq, 82)
