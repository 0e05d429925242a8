"""GPU parity of causal GQA attention forward/backward against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import dev_bf16, host, assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch,seq,nq,nkv,d", [
    (2, 77, 8, 2, 128),     # ragged sequence, two sequences
    (1, 128, 4, 1, 64),
    (2, 64, 7, 1, 64),      # group of 7 (Qwen2.5-0.5B: 14 q / 2 kv heads)
    (1, 96, 8, 1, 128),     # group of 8 (Qwen2.5-3B: 16 q / 2 kv heads)
    (1, 512, 32, 8, 128),   # one Llama-3.1-8B layer at seq 512
    (3, 1, 4, 2, 64),       # one token per sequence
    (1, 2048, 8, 2, 128),   # a long sequence: 32 key tiles in the backward
    (1, 1024, 32, 8, 128),  # the benchmark's layer at 1024 tokens
    (2, 700, 4, 2, 64),     # ragged, two sequences
    (1, 577, 3, 1, 128),    # group of 3, a partly filled last key tile
    (1, 300, 7, 1, 128),    # group of 7 at head_dim 128
    (2, 129, 2, 2, 128),    # one query head per kv head, two sequences, a one-row last key tile
    (1, 33, 2, 1, 128),     # group of 2, a single partial tile
    # more than 512 key tiles in all: dK/dV with one workgroup per key tile (the
    # cases above spread each kv head's dK/dV work evenly over its workgroups)
    (3, 1024, 8, 8, 128),
    (3, 1024, 16, 8, 64),
])
def test_attention_parity(gpu, batch, seq, nq, nkv, d):
    T = batch * seq
    q = synth.activation((T, nq * d), 20 + d, "x", std=1.2)
    k = synth.activation((T, nkv * d), 20 + d, "x", salt=1, std=1.2)
    v = synth.activation((T, nkv * d), 20 + d, "x", salt=2)
    do = synth.activation((T, nq * d), 20 + d, "dy")
    qd, kd, vd, dod = (a.astype(np.float64) for a in (q, k, v, do))
    o_ref, lse_ref = O.attention_fwd(qd.reshape(T, nq, d), kd.reshape(T, nkv, d), vd.reshape(T, nkv, d), batch, seq)
    dq_ref, dk_ref, dv_ref = O.attention_bwd(qd.reshape(T, nq, d), kd.reshape(T, nkv, d), vd.reshape(T, nkv, d),
                                             dod.reshape(T, nq, d), batch, seq)
    Q, K, V, DO = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    o, lse, o32 = gpu.attention_fwd(Q, K, V, batch, seq, nq, nkv, d, want_o32=True)
    dq, dk, dv = gpu.attention_bwd(Q, K, V, o, DO, lse, batch, seq, nq, nkv, d, o32=o32)
    torch.cuda.synchronize()
    assert_close(host(o), o_ref.reshape(T, -1), "attn o")
    assert np.allclose(host(lse), lse_ref, rtol=1e-5, atol=1e-5), np.abs(host(lse) - lse_ref).max()
    assert_close(host(dq), dq_ref.reshape(T, -1), "attn dq")
    assert_close(host(dk), dk_ref.reshape(T, -1), "attn dk")
    assert_close(host(dv), dv_ref.reshape(T, -1), "attn dv")


@pytest.mark.parametrize("d", [64, 128])
def test_attention_strided_views(gpu, d):
    """q, k, v as column slices of one fused qkv row (the layout the layer uses)."""
    batch, seq, nq, nkv = 1, 80, 4, 2
    T, W = batch * seq, (nq + 2 * nkv) * d
    qkv = synth.activation((T, W), 31, "x")
    X = dev_bf16(qkv)
    Q, K, V = X[:, : nq * d], X[:, nq * d:(nq + nkv) * d], X[:, (nq + nkv) * d:]
    o, lse, _ = gpu.attention_fwd(Q, K, V, batch, seq, nq, nkv, d)
    torch.cuda.synchronize()
    qd = qkv.astype(np.float64)
    o_ref, _ = O.attention_fwd(qd[:, : nq * d].reshape(T, nq, d), qd[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d),
                               qd[:, (nq + nkv) * d:].reshape(T, nkv, d), batch, seq)
    assert_close(host(o), o_ref.reshape(T, -1), "attn o (strided)")


def test_attention_forward_is_deterministic(gpu):
    """Repeated forward calls give identical bits (output, its float32 copy and
    the log-sum-exp)."""
    batch, seq, nq, nkv, d = 1, 1024, 8, 2, 128
    T = batch * seq
    g = torch.Generator(device="cuda").manual_seed(7)
    Q = torch.randn(T, nq * d, device="cuda", generator=g).to(torch.bfloat16)
    K = torch.randn(T, nkv * d, device="cuda", generator=g).to(torch.bfloat16)
    V = torch.randn(T, nkv * d, device="cuda", generator=g).to(torch.bfloat16)
    o0, lse0, o320 = gpu.attention_fwd(Q, K, V, batch, seq, nq, nkv, d, want_o32=True)
    for _ in range(3):
        o1, lse1, o321 = gpu.attention_fwd(Q, K, V, batch, seq, nq, nkv, d, want_o32=True)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(lse0, lse1) and torch.equal(o320, o321)


def test_attention_backward_is_deterministic(gpu):
    """Repeated backward calls give identical bits: the Llama-8B layer's shape at
    1024 tokens, whose dK/dV key tiles are split over several workgroups and
    summed in workgroup order by whichever arrives last."""
    batch, seq, nq, nkv, d = 1, 1024, 32, 8, 128
    T = batch * seq
    g = torch.Generator(device="cuda").manual_seed(11)
    Q = torch.randn(T, nq * d, device="cuda", generator=g).to(torch.bfloat16)
    K = torch.randn(T, nkv * d, device="cuda", generator=g).to(torch.bfloat16)
    V = torch.randn(T, nkv * d, device="cuda", generator=g).to(torch.bfloat16)
    DO = torch.randn(T, nq * d, device="cuda", generator=g).to(torch.bfloat16)
    o, lse, o32 = gpu.attention_fwd(Q, K, V, batch, seq, nq, nkv, d, want_o32=True)
    r0 = gpu.attention_bwd(Q, K, V, o, DO, lse, batch, seq, nq, nkv, d, o32=o32)
    for _ in range(3):
        r1 = gpu.attention_bwd(Q, K, V, o, DO, lse, batch, seq, nq, nkv, d, o32=o32)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(r0, r1))
