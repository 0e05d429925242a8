"""Token cross-entropy over the vocabulary from the final hidden states.

The pages measure the naive logits term of the loss ("Exact Layer Streaming ...",
abstract: 14 bytes per logit element against 6 expected). The fused GPU path
never stores logits; what it computes is the plain definition:
  z = h W^T (kept unrounded, as a float accumulator would hold it),
  lse_t = log sum_v exp(z_tv),
  loss = mean over tokens with label != ignore_index of (lse_t - z_t,label),
  dh = rnd(grad_scale / N_valid * (softmax(z) - onehot(label)) W)  (zero rows for ignored tokens).
W (the lm_head or the tied embedding) is frozen, so it gets no gradient.
"""
import numpy as np

from .bf16 import round_bf16


def _logits_lse(h, w):
    z = h @ w.T
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    return z, lse


def ce_loss_fwd(h, w, labels, ignore_index=-100):
    """Returns (loss, lse [T], n_valid)."""
    labels = np.asarray(labels)
    z, lse = _logits_lse(h, w)
    valid = labels != ignore_index
    nv = int(valid.sum())
    if nv == 0:
        return 0.0, lse, 0
    idx = np.nonzero(valid)[0]
    loss = float(np.mean(lse[idx] - z[idx, labels[idx]]))
    return loss, lse, nv


def ce_loss_bwd(h, w, labels, ignore_index=-100, grad_scale=1.0, rnd=round_bf16):
    labels = np.asarray(labels)
    z, lse = _logits_lse(h, w)
    valid = labels != ignore_index
    nv = int(valid.sum())
    p = np.exp(z - lse[:, None])
    idx = np.nonzero(valid)[0]
    p[idx, labels[idx]] -= 1.0
    p[~valid] = 0.0
    if nv:
        p *= grad_scale / nv
    return rnd(p @ w)
