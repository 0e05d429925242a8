"""GPU parity of RMSNorm, RoPE, SwiGLU, embedding gather and AdamW against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import dev_bf16, dev, host, assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,eps", [(37, 4096, 1e-5), (130, 896, 1e-6), (1, 64, 1e-5)])
def test_rmsnorm(gpu, T, H, eps):
    x = synth.activation((T, H), 7, "x")
    dy = synth.activation((T, H), 7, "dy")
    res = synth.activation((T, H), 7, "dy", salt=1)
    w = synth.norm_weight_bf16(H, 7, 0, 0, ones=False)
    y = gpu.rmsnorm_fwd(dev_bf16(x), dev_bf16(w), eps)
    dx = gpu.rmsnorm_bwd(dev_bf16(x), dev_bf16(w), dev_bf16(dy), eps, dres=dev_bf16(res))
    dx0 = gpu.rmsnorm_bwd(dev_bf16(x), dev_bf16(w), dev_bf16(dy), eps)
    torch.cuda.synchronize()
    xd, wd, dyd = x.astype(np.float64), w.astype(np.float64), dy.astype(np.float64)
    assert_close(host(y), O.rmsnorm_fwd(xd, wd, eps), "rmsnorm y")
    assert_close(host(dx), O.round_bf16(res + O.rmsnorm_bwd(xd, wd, eps, dyd)), "rmsnorm dx")
    assert_close(host(dx0), O.round_bf16(O.rmsnorm_bwd(xd, wd, eps, dyd)), "rmsnorm dx (no residual)")


@pytest.mark.parametrize("batch,seq,nh,d,theta", [(2, 40, 3, 128, 500000.0), (1, 1024, 2, 64, 1e6), (3, 7, 1, 16, 1e4)])
def test_rope(gpu, batch, seq, nh, d, theta):
    T = batch * seq
    x = synth.activation((T, nh * d), 8, "x")
    pos = np.tile(np.arange(seq), batch)
    ref = O.rope_apply(x.astype(np.float64).reshape(T, nh, d), pos, theta).reshape(T, nh * d)
    X = dev_bf16(x)
    gpu.rope(X, nh, d, seq, theta)
    torch.cuda.synchronize()
    assert_close(host(X), ref, "rope")
    back = O.rope_apply(x.astype(np.float64).reshape(T, nh, d), pos, theta, inverse=True).reshape(T, nh * d)
    X2 = dev_bf16(x)
    gpu.rope(X2, nh, d, seq, theta, inverse=True)
    torch.cuda.synchronize()
    assert_close(host(X2), back, "rope inverse")


@pytest.mark.parametrize("seq,scaling", [
    (1024, (8.0, 1.0, 4.0, 8192.0)),   # Llama-3.1's published scaling, all three frequency regimes at d 128
    (300, (4.0, 1.0, 2.0, 256.0)),     # positions past the original context, ragged rows
])
def test_rope_llama3_scaling(gpu, seq, scaling):
    T, nh, d, theta = seq, 4, 128, 500000.0
    x = synth.activation((T, nh * d), 11, "x")
    pos = np.arange(seq)
    xd = x.astype(np.float64).reshape(T, nh, d)
    for inverse in (False, True):
        ref = O.rope_apply(xd, pos, theta, inverse=inverse, scaling=scaling).reshape(T, nh * d)
        X = dev_bf16(x)
        gpu.rope(X, nh, d, seq, theta, inverse=inverse, scaling=scaling)
        torch.cuda.synchronize()
        assert_close(host(X), ref, "rope scaled")
        # the rescaled low frequencies really differ from unscaled RoPE
        plain = O.rope_apply(xd, pos, theta, inverse=inverse).reshape(T, nh * d)
        assert np.abs(host(X) - plain).max() > 0.1


def test_rope_strided_heads_leave_other_columns(gpu):
    # q heads inside a wider qkv row: only the first n_heads*d columns change
    T, nh, d, ld = 24, 2, 64, 320
    x = synth.activation((T, ld), 9, "x")
    X = dev_bf16(x)
    gpu.rope(X, nh, d, 24, 1e4)
    torch.cuda.synchronize()
    assert np.array_equal(host(X)[:, nh * d:], x[:, nh * d:])


@pytest.mark.parametrize("T,I", [(33, 4864), (4, 64), (70001, 8)])
def test_swiglu(gpu, T, I):
    gu = synth.activation((T, 2 * I), 10, "x", std=2.0)
    da = synth.activation((T, I), 10, "dy")
    a = gpu.swiglu_fwd(dev_bf16(gu))
    dgu = gpu.swiglu_bwd(dev_bf16(gu), dev_bf16(da))
    torch.cuda.synchronize()
    g, u = gu[:, :I].astype(np.float64), gu[:, I:].astype(np.float64)
    assert_close(host(a), O.swiglu_fwd(g, u), "swiglu a")
    dg, du = O.swiglu_bwd(g, u, da.astype(np.float64))
    assert_close(host(dgu), np.concatenate([dg, du], axis=1), "swiglu dgu")


def test_embed(gpu):
    V, H, T = 1000, 256, 77
    table = synth.normal_bf16((V, H), 0.02, 11, 1000, 50)
    ids = synth.token_ids(T, V, 11)
    out = gpu.embed_fwd(dev_bf16(table), dev(ids))
    torch.cuda.synchronize()
    assert np.array_equal(host(out), table[ids].astype(np.float64))


def test_adamw(gpu):
    n = 10007
    rng = np.random.default_rng(3)
    p0 = rng.standard_normal(n).astype(np.float32)
    P, M, Vv = dev(p0.copy()), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    PB = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    p, m, v = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for step in range(1, 4):
        g = rng.standard_normal(n).astype(np.float32)
        gpu.adamw_step(P, PB, dev(g), M, Vv, step, lr=1e-3, weight_decay=0.01)
        p, m, v = O.adamw_step(p, g.astype(np.float64), m, v, step, lr=1e-3, wd=0.01)
    torch.cuda.synchronize()
    assert np.allclose(host(P), p, rtol=1e-5, atol=1e-6)
    assert_close(host(PB), O.round_bf16(p), "adamw bf16 copy")
