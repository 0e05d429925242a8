"""Token cross-entropy over the vocabulary from the final hidden states.

The pages measure the naive logits term of the loss ("Exact Layer Streaming ...",
abstract: 14 bytes per logit element against 6 expected). The fused GPU path
never stores logits; what it computes is the plain definition:
  z = h W^T (kept unrounded, as a float accumulator would hold it),
  lse_t = log sum_v exp(z_tv),
  loss = mean over tokens with label != ignore_index of (lse_t - z_t,label),
  dh = rnd(grad_scale / N_valid * (softmax(z) - onehot(label)) W)  (zero rows for ignored tokens).
W (the lm_head or the tied embedding) is frozen, so it gets no gradient.

Per-token log-probabilities (the reference model's scores that preference
training compares against, computed with the adapters off on the same streamed
base: "Soup: ...", section on the layer-streaming mechanism, and the news
article's key takeaways on preference training): logp_t = z_t,label - lse_t for
tokens with a label, 0 for ignored ones; a sequence's score is the sum over its
tokens.
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


def ce_token_logprobs(h, w, labels, ignore_index=-100):
    """logp [T] = z_label - lse (0 where the label is ignore_index)."""
    labels = np.asarray(labels)
    z, lse = _logits_lse(h, w)
    out = np.zeros(len(labels))
    idx = np.nonzero(labels != ignore_index)[0]
    out[idx] = z[idx, labels[idx]] - lse[idx]
    return out


def sequence_logprobs(logp, batch, seq):
    """Sum of the token log-probabilities of each sequence [batch]."""
    return np.asarray(logp).reshape(batch, seq).sum(axis=1)
