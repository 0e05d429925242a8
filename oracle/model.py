"""A whole training step of the decoder-only model: embedding gather, the decoder
layers, final RMSNorm, token cross-entropy with shifted labels, the backward
through every layer (recompute), gradient accumulation over microbatches and
AdamW on the adapters.

Streaming changes where the frozen layer weights live, not what is computed
("Exact Layer Streaming ...", abstract: a streamed run must equal a resident run
of the same numerics), so this oracle is the resident computation.
Readings: labels are the next token of the same sequence, the last position of
each sequence is ignored; the embedding table is frozen and resident; the
lm_head is either separate or the tied embedding; every microbatch contributes
loss / n_micro (equal token counts, so this is the mean over all tokens);
gradients are summed in microbatch order.
"""
import numpy as np

from .bf16 import round_bf16
from .ce import ce_loss_fwd, ce_loss_bwd, ce_token_logprobs, sequence_logprobs
from .layer import decoder_layer_fwd, decoder_layer_bwd, rmsnorm_fwd, rmsnorm_bwd

IGNORE = -100


def shifted_labels(ids, batch, seq):
    ids = np.asarray(ids).reshape(batch, seq)
    lab = np.full((batch, seq), IGNORE, np.int64)
    lab[:, :-1] = ids[:, 1:]
    return lab.reshape(-1)


def model_fwd_bwd(ids, emb, final_norm, lm_head, layers, shape, batch, seq,
                  grad_scale=1.0, rnd=round_bf16):
    """One microbatch. layers: list of (w, lora). Returns dict with loss, lse,
    the final hidden hN, the layer-boundary hiddens and per-layer grads."""
    ids = np.asarray(ids)
    wlm = emb if lm_head is None else lm_head
    h = emb[ids]
    hs = [h]
    for w, lora in layers:
        h, _ = decoder_layer_fwd(h, w, lora, shape, batch, seq, rnd)
        hs.append(h)
    hn = rmsnorm_fwd(h, final_norm, shape.rms_eps, rnd)
    labels = shifted_labels(ids, batch, seq)
    loss, lse, nv = ce_loss_fwd(hn, wlm, labels, IGNORE)
    dhn = ce_loss_bwd(hn, wlm, labels, IGNORE, grad_scale, rnd)
    dh = rnd(rmsnorm_bwd(h, final_norm, shape.rms_eps, dhn))
    grads = [None] * len(layers)
    for li in range(len(layers) - 1, -1, -1):
        w, lora = layers[li]
        dh, grads[li] = decoder_layer_bwd(hs[li], dh, w, lora, shape, batch, seq, rnd)
    return {"loss": loss, "lse": lse, "hN": hn, "hiddens": hs, "grads": grads,
            "dh0": dh, "n_valid": nv}


def model_step(id_chunks, emb, final_norm, lm_head, layers, shape, batch, seq, rnd=round_bf16):
    """Gradient accumulation over microbatches (id_chunks: list of [batch*seq] ids).
    Returns (mean loss, accumulated grads per layer, per-microbatch results)."""
    n = len(id_chunks)
    acc = None
    outs = []
    for ids in id_chunks:
        r = model_fwd_bwd(ids, emb, final_norm, lm_head, layers, shape, batch, seq,
                          grad_scale=1.0 / n, rnd=rnd)
        outs.append(r)
        if acc is None:
            acc = [dict(g) for g in r["grads"]]
        else:
            for a, g in zip(acc, r["grads"]):
                for k in a:
                    a[k] = a[k] + g[k]
    loss = sum(o["loss"] for o in outs) / n
    return loss, acc, outs


def reference_logprobs(ids, emb, final_norm, lm_head, layer_weights, shape, batch, seq, rnd=round_bf16):
    """Forward of one microbatch through the base alone (adapters off) and the
    per-token and per-sequence log-probabilities of the shifted labels:
    (logp [batch*seq], seq_logp [batch])."""
    ids = np.asarray(ids)
    wlm = emb if lm_head is None else lm_head
    h = emb[ids]
    for w in layer_weights:
        h, _ = decoder_layer_fwd(h, w, None, shape, batch, seq, rnd)
    hn = rmsnorm_fwd(h, final_norm, shape.rms_eps, rnd)
    logp = ce_token_logprobs(hn, wlm, shifted_labels(ids, batch, seq), IGNORE)
    return logp, sequence_logprobs(logp, batch, seq)
