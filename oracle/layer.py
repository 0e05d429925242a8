"""One pre-norm decoder layer (Llama / Qwen2 shape): RMSNorm, RoPE, GQA causal
attention, SwiGLU MLP, residual adds, with LoRA on all seven projections.

The pages stream "decoder layers" of Llama-3.1-8B and Qwen2.5 bases through the
forward and the backward pass ("Soup CLI ...", section "How Layer Streaming
Works"); the layer itself is the published architecture of those bases:
  * RMSNorm (Zhang & Sennrich 2019): y = x / sqrt(mean(x^2) + eps) * w;
  * rotary embedding, rotate-half form (Su et al. 2021, RoFormer section 3.4;
    the halves x[:d/2], x[d/2:] form the rotated pairs), angle = pos * theta^(-2i/d),
    positions restart at 0 in every sequence of the batch;
  * grouped-query causal attention (Ainslie et al. 2023): query head h reads
    kv head h // (n_q / n_kv); scores scaled by 1/sqrt(d); key j visible to
    query i iff j <= i within the same sequence;
  * SwiGLU MLP (Shazeer 2020): down(silu(gate(x)) * up(x)).
  * h' = x + o(attn(...)); out = h' + down(...).
Model-fidelity options (off unless the shape asks for them):
  * q/k/v bias (Qwen2 bases): frozen bf16 vectors added to those three
    projections before their single rounding; no gradient;
  * Llama-3.1 RoPE frequency scaling (the rope_type "llama3" configuration
    published with Llama-3.1: factor, low/high frequency factors and the
    original context length): inverse frequencies whose wavelength 2 pi / f is
    shorter than original / high_factor stay; those longer than
    original / low_factor are divided by factor; in between the two are blended
    linearly in original / wavelength.
Reading: the backward recomputes the forward from the layer input (nothing but
the layer input is kept).

bf16 mode rounds (with rnd) every tensor the GPU path stores in bfloat16; all
arithmetic is float64.
"""
import numpy as np

from .bf16 import round_bf16
from .lora import lora_linear_fwd, lora_linear_bwd, base_linear_fwd


# ---------------------------------------------------------------- RMSNorm
def rmsnorm_fwd(x, w, eps, rnd=round_bf16):
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return rnd(x * r * w)


def rmsnorm_bwd(x, w, eps, dy):
    """dx = r (w*dy - xh * mean(xh * w * dy)),  xh = x r  (unrounded)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xh = x * r
    g = w * dy
    return r * (g - xh * np.mean(xh * g, axis=-1, keepdims=True))


# ---------------------------------------------------------------- RoPE
def rope_inv_freq(head_dim, theta, scaling=None):
    """Inverse frequencies theta^(-2i/d), i < d/2; scaling = (factor,
    low_freq_factor, high_freq_factor, original_max_position) or None."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / head_dim)
    if scaling is None:
        return inv
    factor, low, high, orig = (float(v) for v in scaling)
    out = np.empty_like(inv)
    for j, f in enumerate(inv):
        wavelen = 2.0 * np.pi / f
        if wavelen < orig / high:          # high frequencies: unchanged
            out[j] = f
        elif wavelen > orig / low:         # low frequencies: slowed by factor
            out[j] = f / factor
        else:                              # the band between: linear blend in orig / wavelen
            mix = (orig / wavelen - low) / (high - low)
            out[j] = (1.0 - mix) * f / factor + mix * f
    return out


def rope_angles(positions, head_dim, theta, scaling=None):
    inv = rope_inv_freq(head_dim, theta, scaling)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]


def rope_apply(x, positions, theta, inverse=False, rnd=round_bf16, scaling=None):
    """x [T x heads x d]; rotate pairs (x[i], x[i + d/2]) by +angle (or -angle)."""
    d = x.shape[-1]
    ang = rope_angles(positions, d, theta, scaling)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return rnd(np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1))


def positions_of(batch, seq):
    return np.tile(np.arange(seq), batch)


# ---------------------------------------------------------------- attention
def _split(x, batch, seq):
    return x.reshape(batch, seq, x.shape[1], x.shape[2])


def attention_fwd(q, k, v, batch, seq, rnd=round_bf16):
    """q [T x nq x d], k, v [T x nkv x d] -> (O [T x nq x d], lse [batch x nq x seq])."""
    nq, d = q.shape[1], q.shape[2]
    nkv = k.shape[1]
    grp = nq // nkv
    qb, kb, vb = _split(q, batch, seq), _split(k, batch, seq), _split(v, batch, seq)
    o = np.zeros_like(qb)
    lse = np.zeros((batch, nq, seq))
    mask = np.triu(np.ones((seq, seq), bool), 1)
    for b in range(batch):
        for h in range(nq):
            g = h // grp
            s = (qb[b, :, h, :] @ kb[b, :, g, :].T) / np.sqrt(d)
            s[mask] = -np.inf
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            o[b, :, h, :] = (p / l) @ vb[b, :, g, :]
            lse[b, h] = (m + np.log(l))[:, 0]
    return rnd(o.reshape(q.shape)), lse


def attention_bwd(q, k, v, do, batch, seq, rnd=round_bf16):
    """Gradients (dq, dk, dv) of sum(do * attention(q, k, v)); dk, dv summed over each group."""
    nq, d = q.shape[1], q.shape[2]
    nkv = k.shape[1]
    grp = nq // nkv
    qb, kb, vb, dob = (_split(t, batch, seq) for t in (q, k, v, do))
    dq = np.zeros_like(qb)
    dk = np.zeros_like(kb)
    dv = np.zeros_like(vb)
    mask = np.triu(np.ones((seq, seq), bool), 1)
    sc = 1.0 / np.sqrt(d)
    for b in range(batch):
        for h in range(nq):
            g = h // grp
            s = (qb[b, :, h, :] @ kb[b, :, g, :].T) * sc
            s[mask] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = dob[b, :, h, :] @ vb[b, :, g, :].T
            dsum = np.sum(p * dp, axis=1, keepdims=True)
            ds = p * (dp - dsum)
            dq[b, :, h, :] = (ds @ kb[b, :, g, :]) * sc
            dk[b, :, g, :] += (ds.T @ qb[b, :, h, :]) * sc
            dv[b, :, g, :] += p.T @ dob[b, :, h, :]
    return rnd(dq.reshape(q.shape)), rnd(dk.reshape(k.shape)), rnd(dv.reshape(v.shape))


# ---------------------------------------------------------------- SwiGLU
def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def swiglu_fwd(g, u, rnd=round_bf16):
    return rnd(g * _sigmoid(g) * u)


def swiglu_bwd(g, u, da, rnd=round_bf16):
    sg = _sigmoid(g)
    dg = da * u * sg * (1.0 + g * (1.0 - sg))
    du = da * g * sg
    return rnd(dg), rnd(du)


# ---------------------------------------------------------------- decoder layer
def decoder_layer_fwd(x, w, lora, shape, batch, seq, rnd=round_bf16):
    """Forward of one layer. w: dequantised weights ('q','k','v','o','gate','up','down'
    [out x in], 'norm1', 'norm2'); lora: 'A_p' [r x in], 'B_p' [out x r], or None
    for the base alone (adapters off).
    Returns (out, cache) where cache holds every intermediate the backward needs."""
    s = shape.lora_scale

    def proj(xx, p, bias=None):
        if lora is None:
            return base_linear_fwd(xx, w[p], rnd, bias), None
        return lora_linear_fwd(xx, w[p], lora["A_" + p], lora["B_" + p], s, rnd, bias=bias)

    nq, nkv, d = shape.n_q, shape.n_kv, shape.head_dim
    T = x.shape[0]
    pos = positions_of(batch, seq)
    c = {"x": x}
    c["n1"] = n1 = rmsnorm_fwd(x, w["norm1"], shape.rms_eps, rnd)
    sc = getattr(shape, "rope_scaling", None)
    for p in ("q", "k", "v"):
        c[p], c["t_" + p] = proj(n1, p, bias=w.get(p + "_bias"))
    c["qr"] = rope_apply(c["q"].reshape(T, nq, d), pos, shape.rope_theta, rnd=rnd, scaling=sc)
    c["kr"] = rope_apply(c["k"].reshape(T, nkv, d), pos, shape.rope_theta, rnd=rnd, scaling=sc)
    vv = c["v"].reshape(T, nkv, d)
    o, c["lse"] = attention_fwd(c["qr"], c["kr"], vv, batch, seq, rnd)
    c["attn"] = o = o.reshape(T, nq * d)
    c["o"], c["t_o"] = proj(o, "o")
    c["h1"] = h1 = rnd(x + c["o"])
    c["n2"] = n2 = rmsnorm_fwd(h1, w["norm2"], shape.rms_eps, rnd)
    for p in ("gate", "up"):
        c[p], c["t_" + p] = proj(n2, p)
    c["act"] = a = swiglu_fwd(c["gate"], c["up"], rnd)
    c["down"], c["t_down"] = proj(a, "down")
    out = rnd(h1 + c["down"])
    return out, c


def decoder_layer_bwd(x, dout, w, lora, shape, batch, seq, rnd=round_bf16):
    """Backward with recompute: rebuilds the forward from x, then returns
    (dx, grads) with grads['A_p'] [r x in], grads['B_p'] [out x r] (unrounded)."""
    s = shape.lora_scale
    nq, nkv, d = shape.n_q, shape.n_kv, shape.head_dim
    T = x.shape[0]
    pos = positions_of(batch, seq)
    _, c = decoder_layer_fwd(x, w, lora, shape, batch, seq, rnd)
    gr = {}
    # MLP
    da, gr["A_down"], gr["B_down"], _ = lora_linear_bwd(
        c["act"], c["t_down"], dout, w["down"], lora["A_down"], lora["B_down"], s, rnd)
    dg, du = swiglu_bwd(c["gate"], c["up"], da, rnd)
    dn2 = 0.0
    for p, dp in (("gate", dg), ("up", du)):
        dxp, gr["A_" + p], gr["B_" + p], _ = lora_linear_bwd(
            c["n2"], c["t_" + p], dp, w[p], lora["A_" + p], lora["B_" + p], s, rnd, round_dx=False)
        dn2 = dn2 + dxp
    dn2 = rnd(dn2)
    dh1 = rnd(dout + rmsnorm_bwd(c["h1"], w["norm2"], shape.rms_eps, dn2))
    # attention block
    dattn, gr["A_o"], gr["B_o"], _ = lora_linear_bwd(
        c["attn"], c["t_o"], dh1, w["o"], lora["A_o"], lora["B_o"], s, rnd)
    dqr, dkr, dv = attention_bwd(c["qr"], c["kr"], c["v"].reshape(T, nkv, d),
                                 dattn.reshape(T, nq, d), batch, seq, rnd)
    sc = getattr(shape, "rope_scaling", None)
    dq = rope_apply(dqr, pos, shape.rope_theta, inverse=True, rnd=rnd, scaling=sc).reshape(T, nq * d)
    dk = rope_apply(dkr, pos, shape.rope_theta, inverse=True, rnd=rnd, scaling=sc).reshape(T, nkv * d)
    dv = dv.reshape(T, nkv * d)
    dn1 = 0.0
    for p, dp in (("q", dq), ("k", dk), ("v", dv)):
        dxp, gr["A_" + p], gr["B_" + p], _ = lora_linear_bwd(
            c["n1"], c["t_" + p], dp, w[p], lora["A_" + p], lora["B_" + p], s, rnd, round_dx=False)
        dn1 = dn1 + dxp
    dn1 = rnd(dn1)
    dx = rnd(dh1 + rmsnorm_bwd(x, w["norm1"], shape.rms_eps, dn1))
    return dx, gr
