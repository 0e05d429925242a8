"""GPU parity of the fused, vocabulary-chunked cross-entropy against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import dev_bf16, dev, host, assert_close_chain, assert_close_scaled

pytestmark = pytest.mark.gpu


def _case(T, H, V, wid, n_ignore=3):
    h = synth.activation((T, H), wid, "x")
    w = synth.normal_bf16((V, H), 0.05, wid, 1000, 52)
    labels = synth.token_ids(T, V, wid).astype(np.int64)
    labels[np.arange(n_ignore) * 7 % T] = -100
    return h, w, labels


@pytest.mark.parametrize("T,H,V,gs", [
    (100, 128, 69952, 1.0),     # three vocabulary chunks of the backward, the last one partial; ragged T
    # 256 x 256 tiles: the forward logits, the first gradient chunk (the second,
    # 7232 columns, in 64-row tiles) and the dH accumulation with 8 reduction
    # splits; two token tiles, the second ragged; a partial vocabulary tile
    (300, 4096, 40000, 1.0),
    (100, 128, 16576, 1.0),     # one chunk, a partial vocabulary tile
    (37, 256, 1088, 0.25),      # one chunk with a partial vocabulary tile, a gradient scale
    (1, 64, 64, 1.0),
])
def test_ce_parity(gpu, T, H, V, gs):
    h, w, labels = _case(T, H, V, 50 + T)
    hd, wd = h.astype(np.float64), w.astype(np.float64)
    loss_ref, lse_ref, nv = O.ce_loss_fwd(hd, wd, labels)
    dh_ref = O.ce_loss_bwd(hd, wd, labels, grad_scale=gs)
    Hh, W, L = dev_bf16(h), dev_bf16(w), dev(labels.astype(np.int32))
    loss, lse = gpu.fused_ce_loss_fwd(Hh, W, L)
    dh = gpu.fused_ce_loss_bwd(Hh, W, L, lse, grad_scale=gs)
    torch.cuda.synchronize()
    assert abs(loss.item() - loss_ref) <= 1e-5 * abs(loss_ref), (loss.item(), loss_ref)
    assert np.allclose(host(lse), lse_ref, rtol=1e-5, atol=0)
    # dh is O(grad_scale / N_valid): the per-element bound with its absolute term
    # scaled to the tensor (the plain 1e-2 would be vacuous at that size)
    assert_close_scaled(host(dh), dh_ref, "ce dh")
    assert_close_chain(host(dh), dh_ref, "ce dh (scale-free)")
    assert_close_chain(host(dh) * nv, dh_ref * nv, "ce dh * N_valid")


def test_ce_zero_weights_closed_form(gpu):
    T, H, V = 50, 128, 4096
    h, _, labels = _case(T, H, V, 61)
    W = torch.zeros((V, H), dtype=torch.bfloat16, device="cuda")
    loss, lse = gpu.fused_ce_loss_fwd(dev_bf16(h), W, dev(labels.astype(np.int32)))
    dh = gpu.fused_ce_loss_bwd(dev_bf16(h), W, dev(labels.astype(np.int32)), lse)
    torch.cuda.synchronize()
    assert abs(loss.item() - math.log(V)) < 1e-5 * math.log(V)
    assert np.allclose(host(lse), math.log(V), rtol=1e-6)
    assert torch.count_nonzero(dh) == 0


def test_ce_all_ignored(gpu):
    T, H, V = 16, 64, 128
    h, w, _ = _case(T, H, V, 62)
    labels = np.full(T, -100, np.int32)
    loss, lse = gpu.fused_ce_loss_fwd(dev_bf16(h), dev_bf16(w), dev(labels))
    dh = gpu.fused_ce_loss_bwd(dev_bf16(h), dev_bf16(w), dev(labels), lse)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and torch.count_nonzero(dh) == 0


@pytest.mark.timeout(900)
def test_ce_llama8b_head_sampled_rows(gpu):
    """Full Llama-3.1-8B head (1024 tokens, hidden 4096, vocab 128256) on the GPU;
    the oracle checks 48 sampled tokens (each token's lse and dh row depend only
    on its own row and on the number of valid labels)."""
    T, H, V = 1024, 4096, 128256
    h = synth.activation((T, H), 5, "x")
    w = synth.normal_bf16((V, H), 0.02, 5, 1000, 52)
    labels = synth.token_ids(T, V, 5).astype(np.int64)
    labels[T - 1] = -100
    Hh, W, L = dev_bf16(h), dev_bf16(w), dev(labels.astype(np.int32))
    loss, lse = gpu.fused_ce_loss_fwd(Hh, W, L)
    dh = gpu.fused_ce_loss_bwd(Hh, W, L, lse)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(0).choice(T, 48, replace=False))
    rows[-1] = T - 1
    hd, wd = h[rows].astype(np.float64), w.astype(np.float64)
    _, lse_ref, _ = O.ce_loss_fwd(hd, wd, labels[rows])
    nv_all = int(np.sum(labels != -100))
    dh_ref = O.ce_loss_bwd(hd, wd, labels[rows], grad_scale=len(np.nonzero(labels[rows] != -100)[0]) / nv_all)
    assert np.allclose(host(lse)[rows], lse_ref, rtol=1e-5, atol=0)
    assert_close_scaled(host(dh)[rows], dh_ref, "ce dh rows")
    assert_close_chain(host(dh)[rows] * nv_all, dh_ref * nv_all, "ce dh rows * N_valid")
    assert np.all(host(dh)[T - 1] == 0)


@pytest.mark.parametrize("T,H,V,batch", [
    (100, 128, 16576, 4),       # ragged vocabulary tile, 4 sequences of 25
    (100, 128, 69952, 2),       # forward logits in 256 x 256 tiles, a partial one at the end
    (37, 256, 1088, 1),
    (1, 64, 64, 1),
])
def test_ce_logprobs_parity(gpu, T, H, V, batch):
    """Per-token log-probabilities z_label - lse (0 where ignored) and their
    per-sequence sums. float32 outputs: |gpu - oracle| <= 1e-5 (|z_label| +
    |lse|) per token (the float32 loss bound applied to each of the two terms),
    and the sum of those bounds per sequence."""
    from oracle.ce import ce_token_logprobs, sequence_logprobs
    h, w, labels = _case(T, H, V, 70 + T)
    hd, wd = h.astype(np.float64), w.astype(np.float64)
    lp_ref = ce_token_logprobs(hd, wd, labels)
    _, lse_ref, _ = O.ce_loss_fwd(hd, wd, labels)
    bound = 1e-5 * (np.abs(lp_ref + lse_ref) + np.abs(lse_ref)) + 1e-7
    bound[labels == -100] = 0.0
    lp, slp = gpu.fused_ce_logprobs(dev_bf16(h), dev_bf16(w), dev(labels.astype(np.int32)), batch)
    torch.cuda.synchronize()
    err = np.abs(host(lp) - lp_ref)
    assert np.all(err <= bound), (err.max(), np.argmax(err - bound))
    assert np.all(host(lp)[labels == -100] == 0)
    sb = bound.reshape(batch, -1).sum(1) + 1e-6 * np.abs(sequence_logprobs(lp_ref, batch, T // batch))
    assert np.all(np.abs(host(slp) - sequence_logprobs(lp_ref, batch, T // batch)) <= sb)
    # same bits as minus the training forward's per-token loss terms: the two share the same pass
    loss, _ = gpu.fused_ce_loss_fwd(dev_bf16(h), dev_bf16(w), dev(labels.astype(np.int32)))
    torch.cuda.synchronize()
    nv = int(np.sum(labels != -100))
    if nv:
        assert abs(loss.item() + host(lp).sum() / nv) <= 1e-5 * abs(loss.item()) + 1e-6
