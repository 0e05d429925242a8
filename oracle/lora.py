"""LoRA linear: y = x W^T + s (x A^T) B^T with a frozen W and trainable A [r x in], B [out x r].

The pages train low-rank adapters on a frozen base ("Exact Layer Streaming ...",
abstract; "Soup CLI ...", "How Layer Streaming Works": the base stays frozen).
The adapter form y = x W^T + (alpha/r) x A^T B^T is the standard LoRA
parametrisation (Hu et al. 2021, section 4.1); no dropout (reading).

bf16 mode rounds t = x A^T, u = dy B and the outputs y, dx once each; the
adapter gradients are float outputs (no rounding). W has no gradient.
"""
import numpy as np

from .bf16 import round_bf16


def lora_linear_fwd(x, w, a, b, scale, rnd=round_bf16, bias=None):
    """Returns (y, t). x [T x in], w [out x in], a [r x in], b [out x r].
    bias [out] (optional, frozen like W: the q/k/v projections of Qwen2 bases)
    joins the sum before the single rounding of y."""
    t = rnd(x @ a.T)
    y = x @ w.T + scale * (t @ b.T)
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return rnd(y), t


def base_linear_fwd(x, w, rnd=round_bf16, bias=None):
    """The frozen projection alone (adapters off): y = rnd(x W^T (+ bias))."""
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return rnd(y)


def lora_adapter_grads(x, t, dy, u, scale):
    """The adapter gradients of one LoRA linear from its forward input x,
    t = x A^T, the loss gradient dy and u = dy B: dA = s u^T x, dB = s dy^T t
    (unrounded; the chain rule through y = x W^T + s t B^T with t = x A^T)."""
    return scale * (u.T @ x), scale * (dy.T @ t)


def lora_linear_bwd(x, t, dy, w, a, b, scale, rnd=round_bf16, round_dx=True):
    """Returns (dx, dA, dB, u) for the loss gradient dy [T x out].

    dx = dy W + s (dy B) A;  dA = s (dy B)^T x;  dB = s dy^T t.
    With round_dx=False dx is returned unrounded so callers can sum several
    projections that read the same input before rounding once.
    """
    u = rnd(dy @ b)
    dx = dy @ w + scale * (u @ a)
    if round_dx:
        dx = rnd(dx)
    da, db = lora_adapter_grads(x, t, dy, u, scale)
    return dx, da, db, u
