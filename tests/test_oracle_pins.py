"""Pins of the CPU oracle to things other than itself: library routines (torch
CPU float64 ops, scipy), closed forms, brute force on tiny inputs, invariants
and central finite differences. A plausible slip in the oracle (a dropped term,
a wrong sign, a transposed operand, a wrong head mapping) fails one of these."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from oracle.bf16 import round_bf16, identity, bf16_bits, from_bf16_bits
from oracle.nf4 import nf4_codebook, nf4_quantize, nf4_dequant, nf4_unpack
from oracle.nf4 import nf4dq_quantize, nf4dq_quantize_absmax, nf4dq_absmax, nf4dq_dequant, nf4dq_layer_bytes
from oracle.nf4 import nf4dq_quantize_fused
from synth.configs import TINY_LAYER, PROJ_IN_OUT

RNG = np.random.default_rng(1234)
GOLDEN = __import__('os').path.join(__import__('os').path.dirname(__file__), 'golden')


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# ------------------------------------------------------------------ bf16
def test_bf16_matches_torch_conversion():
    x = np.concatenate([RNG.standard_normal(20000) * 10.0 ** RNG.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16_bits(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6 (even)
    assert round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -20]))[0] == 1.0 + 2.0 ** -7
    assert np.isnan(round_bf16(np.array([np.nan]))[0])
    assert np.array_equal(from_bf16_bits(np.array([0x3F80, 0xC000], np.uint16)), [1.0, -2.0])


# ------------------------------------------------------------------ NF4
def test_nf4_codebook_invariants():
    cb = nf4_codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[7] == 0.0 and cb[15] == 1.0
    assert np.sum(cb < 0) == 7 and np.sum(cb > 0) == 8


def test_nf4_codebook_is_normal_quantiles():
    """Each code value times Phi^-1(delta) maps back (through scipy's normal CDF)
    onto the evenly spaced probability grid of the NormalFloat construction."""
    from scipy.stats import norm
    cb = nf4_codebook().astype(np.float64)
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    top = norm.ppf(delta)
    pos_p = norm.cdf(cb[8:] * top)          # ascending
    neg_p = norm.cdf(-cb[:7] * top)         # for negated values, ascending after reversal
    assert np.allclose(np.sort(pos_p), np.linspace(delta, 0.5, 9)[:-1][::-1], atol=2e-7)
    assert np.allclose(np.sort(neg_p), np.linspace(delta, 0.5, 8)[:-1][::-1], atol=2e-7)
    # scipy's ppf gives the same float32 table
    v = sorted(list(norm.ppf(np.linspace(delta, 0.5, 9)[:-1])) +
               list(-norm.ppf(np.linspace(delta, 0.5, 8)[:-1])) + [0.0])
    assert np.array_equal((np.array(v) / max(v)).astype(np.float32), nf4_codebook())


def _brute_codes(w):
    cb = nf4_codebook()
    f = w.astype(np.float32).reshape(-1, 64)
    out = np.empty(f.shape, np.uint8)
    am = np.abs(f).max(axis=1)
    for b in range(f.shape[0]):
        for i in range(64):
            n = np.float32(0.0) if am[b] == 0 else np.float32(f[b, i] / am[b])
            d = [abs(float(n) - float(c)) for c in cb]
            best = min(d)
            # nearest; on an exact tie the lower index
            out[b, i] = [j for j in range(16) if d[j] == best][0]
    return out.reshape(w.shape), am


def test_nf4_quantize_brute_force():
    w = round_bf16(RNG.standard_normal((4, 128)) * 0.02)
    w[1, :64] = 0.0                      # all-zero block
    w[2, 64:] = 0.0
    w[2, 70] = -0.5                      # single non-zero (negative) element
    packed, absmax = nf4_quantize(w)
    codes = nf4_unpack(packed)
    bc, bam = _brute_codes(w)
    assert np.array_equal(absmax.reshape(-1), bam)
    # exact ties (n equal to a float32 midpoint) are the only place nearest can differ
    assert np.array_equal(codes, bc)
    assert np.all(codes[1, :64] == 7)
    assert codes[2, 70] == 0 and np.all(codes[2, 64:70] == 7)


def test_nf4_midpoint_ties_go_low():
    cb = nf4_codebook()
    mids = ((cb[:-1] + cb[1:]) * np.float32(0.5)).astype(np.float32)
    # a block whose absmax is 1 makes n == w exactly
    for i in (0, 6, 7, 12):
        blk = np.zeros(64)
        blk[0] = 1.0
        blk[1] = float(mids[i])
        if round_bf16(np.array([blk[1]]))[0] != blk[1]:
            continue                     # only bf16-representable midpoints can occur
        c = nf4_unpack(nf4_quantize(blk[None, :])[0])[0]
        assert c[1] == i


def test_nf4_pack_order_and_roundtrip():
    blk = np.zeros((1, 64))
    blk[0, 0], blk[0, 1] = 1.0, -1.0
    packed, absmax = nf4_quantize(blk)
    assert packed[0, 0] == 0xF0 and packed[0, 1] == 0x77 and absmax[0, 0] == 1.0
    w = round_bf16(RNG.standard_normal((8, 256)) * 0.05)
    packed, absmax = nf4_quantize(w)
    deq32 = nf4_dequant(packed, absmax, rnd=identity)
    ratio = deq32.reshape(-1, 64) / absmax.reshape(-1, 1).astype(np.float64)
    cb = nf4_codebook().astype(np.float64)
    # dequant(quant(w)) / absmax is a code value (exact float32 product, no rounding)
    assert np.all(np.isin(np.round(ratio, 6), np.round(cb, 6)))
    # the element holding absmax comes back exactly
    deq = nf4_dequant(packed, absmax)
    fb = np.abs(w.reshape(-1, 64))
    am_idx = fb.argmax(axis=1)
    got = np.abs(deq.reshape(-1, 64)[np.arange(fb.shape[0]), am_idx])
    assert np.array_equal(got, fb.max(axis=1))
    # quant o dequant o quant == quant
    p2, a2 = nf4_quantize(deq)
    assert np.array_equal(p2, packed) and np.array_equal(a2, absmax)


def test_nf4_dequant_single_fp32_multiply():
    w = round_bf16(RNG.standard_normal((2, 64)) * 0.02)
    packed, absmax = nf4_quantize(w)
    codes = nf4_unpack(packed)
    cb = nf4_codebook()
    exp = (torch.from_numpy(cb[codes]) * torch.from_numpy(absmax.repeat(64, axis=1))).to(torch.bfloat16)
    assert np.array_equal(nf4_dequant(packed, absmax), exp.double().numpy())


# ------------------------------------------------------------------ finite differences
def fd_grad(f, x, idx_list, eps=1e-6):
    out = []
    for idx in idx_list:
        xp = x.copy(); xp[idx] += eps
        xm = x.copy(); xm[idx] -= eps
        out.append((f(xp) - f(xm)) / (2 * eps))
    return np.array(out)


def sample_idx(shape, n, rng):
    return [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(n)]


def assert_fd(analytic, f, x, n=12, rtol=1e-6, atol=1e-9):
    rng = np.random.default_rng(7)
    idx = sample_idx(x.shape, n, rng)
    num = fd_grad(f, x, idx)
    ana = np.array([analytic[i] for i in idx])
    # central differences carry roundoff of about 1e-16 * |f| / eps
    atol = atol + 1e-7 * max(1.0, float(np.max(np.abs(num))))
    assert np.allclose(ana, num, rtol=rtol, atol=atol), (ana, num)


# ------------------------------------------------------------------ NF4 double quantisation
def test_nf4dq_store_sizes_match_the_pages():
    """The page's pre-flight sizes for Llama-3.1-8B (tests/golden/pages_store_sizes.json)
    are those of 4-bit codes + 8-bit absmax + one float32 per 256 absmax values."""
    import json
    g = json.load(open(__import__("os").path.join(GOLDEN, "pages_store_sizes.json")))
    m = g["model"]
    b = nf4dq_layer_bytes(m["hidden"], m["n_q"], m["n_kv"], m["head_dim"], m["inter"])
    assert round(b / 1e6) == g["buffer_MB"]
    assert round(m["layers"] * b / 1e9, 2) == g["store_GB"]
    # float32 absmax (one per 64 weights) would not fit those sizes
    fp32_absmax = b + sum(n * k // 64 * 3 for n, k in [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
                                                       (14336, 4096), (14336, 4096), (4096, 14336)])
    assert round(m["layers"] * fp32_absmax / 1e9, 2) != g["store_GB"]


def _brute_q(a, s):
    """Nearest integer in [0, 255] to a / s in exact arithmetic (ties to even)."""
    out = np.zeros(a.size, np.int64)
    for i, v in enumerate(a.astype(np.float64)):
        if s == 0:
            continue
        x = v / float(s)
        best = min(range(256), key=lambda q: (abs(q - x), q % 2))
        out[i] = best
    return out


def test_nf4dq_absmax_brute_force_and_bounds():
    a = np.abs(RNG.standard_normal(600) * 0.03).astype(np.float32)   # blocks of 256, 256, 88
    a[256:512] = 0.0                                                   # an all-zero block
    a[300] = 0.0
    q, s = nf4dq_quantize_absmax(a.reshape(6, 100))
    q = q.reshape(-1)
    assert s.shape == (3,) and s[1] == 0.0 and np.all(q[256:512] == 0)
    for b in range(3):
        blk = a[b * 256:(b + 1) * 256]
        assert s[b] == np.float32(np.max(blk) / np.float32(255.0))
        assert np.array_equal(q[b * 256:(b + 1) * 256], _brute_q(blk, s[b]))
        if s[b] > 0:
            assert q[b * 256 + int(np.argmax(blk))] == 255
    a2 = nf4dq_absmax(q.reshape(6, 100), s).reshape(-1).astype(np.float64)
    err = np.abs(a2 - a)
    bound = np.repeat(s.astype(np.float64), 256)[:600] * (0.5 + 1e-5)
    assert np.all(err <= bound)


def test_nf4dq_dequant_values_and_error():
    w = round_bf16(RNG.standard_normal((32, 512)) * 0.02)
    w[3, :] = 0.0
    packed, q, s = nf4dq_quantize(w)
    p2, absmax = nf4_quantize(w)
    assert np.array_equal(packed, p2)                       # codes chosen with the exact absmax
    deq = nf4dq_dequant(packed, q, s, rnd=identity)
    a2 = nf4dq_absmax(q, s).reshape(-1).astype(np.float64)
    ratio = deq.reshape(-1, 64) / np.where(a2 > 0, a2, 1.0)[:, None]
    cb = nf4_codebook().astype(np.float64)
    assert np.all(np.isin(np.round(ratio, 5), np.round(cb, 5)))   # every value is code * absmax'
    assert np.all(deq[3] == 0.0)
    # error: NF4 rounding (half the widest code gap) plus the absmax error
    gap = np.max(np.diff(cb)) / 2
    tol = absmax.reshape(-1, 1) * gap + np.repeat(s, 256)[:absmax.size].reshape(-1, 1) * 0.5 * 1.0001
    assert np.all(np.abs(deq - w).reshape(-1, 64) <= tol + 1e-12)


def test_nf4dq_fused_equals_separate_on_whole_blocks():
    """Stacked matrices whose absmax counts are multiples of 256 (rows x cols both
    multiples of 128) double-quantize exactly as each matrix alone."""
    mats = [round_bf16(RNG.standard_normal((r, 256)) * sd) for r, sd in ((128, 0.02), (64 * 2, 0.5), (128, 0.001))]
    fused = nf4dq_quantize_fused(mats)
    for m, f in zip(mats, fused):
        assert np.array_equal(f, nf4dq_dequant(*nf4dq_quantize(m)))


def test_nf4dq_fused_block_straddles_matrices():
    """With 64 x 320 (320 absmax, not a multiple of 256) on top of a matrix of a
    much larger scale, the second 256-block holds the tail of the first matrix
    and the head of the second: its constant is the largest absmax of both
    parts / 255, so the small matrix's tail loses precision that quantizing it
    alone keeps."""
    a = round_bf16(RNG.standard_normal((64, 320)) * 0.001)
    b = round_bf16(RNG.standard_normal((64, 320)) * 1.0)
    fa, fb = nf4dq_quantize_fused([a, b])
    assert np.array_equal(fa[:51], nf4dq_dequant(*nf4dq_quantize(a))[:51])   # rows 0..50 sit in block 0 only
    _, absmax_b = nf4_quantize(b)
    _, absmax_a = nf4_quantize(a)
    s1 = np.float32(max(absmax_a.reshape(-1)[256:].max(), absmax_b.reshape(-1)[:192].max()) / np.float32(255.0))
    _, q, scale = nf4dq_quantize(np.concatenate([a, b], 0))
    assert scale[1] == s1
    # a's tail shares block 1 with b's head: fused and separate differ for a
    assert not np.array_equal(fa, nf4dq_dequant(*nf4dq_quantize(a)))


# ------------------------------------------------------------------ LoRA linear
def _lora_inputs(T=6, fin=64, fout=32, r=4):
    x = RNG.standard_normal((T, fin))
    w = RNG.standard_normal((fout, fin)) * 0.1
    a = RNG.uniform(-0.2, 0.2, (r, fin))
    b = RNG.standard_normal((fout, r)) * 0.1
    return x, w, a, b


def test_lora_zero_b_is_plain_linear():
    x, w, a, _ = _lora_inputs()
    xb, wb, ab = round_bf16(x), round_bf16(w), round_bf16(a)
    y, _ = O.lora_linear_fwd(xb, wb, ab, np.zeros((32, 4)), 2.0)
    ref = F.linear(t64(xb), t64(wb)).to(torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(y, ref)


def test_lora_merged_weight_identity():
    x, w, a, b = _lora_inputs()
    y, _ = O.lora_linear_fwd(x, w, a, b, 2.0, rnd=identity)
    ref = F.linear(t64(x), t64(w) + 2.0 * (t64(b) @ t64(a))).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_lora_bwd_finite_differences():
    x, w, a, b = _lora_inputs()
    dy = RNG.standard_normal((6, 32))
    s = 2.0
    y, t = O.lora_linear_fwd(x, w, a, b, s, rnd=identity)
    dx, da, db, _ = O.lora_linear_bwd(x, t, dy, w, a, b, s, rnd=identity)
    L = lambda **kw: float(np.sum(dy * O.lora_linear_fwd(kw.get("x", x), w, kw.get("a", a), kw.get("b", b), s, rnd=identity)[0]))
    assert_fd(dx, lambda v: L(x=v), x)
    assert_fd(da, lambda v: L(a=v), a)
    assert_fd(db, lambda v: L(b=v), b)


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_matches_torch():
    x = RNG.standard_normal((5, 48))
    w = 1 + RNG.uniform(-0.1, 0.1, 48)
    y = O.rmsnorm_fwd(x, w, 1e-5, rnd=identity)
    ref = F.rms_norm(t64(x), (48,), t64(w), eps=1e-5).numpy()
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_rmsnorm_bwd_fd_and_invariance():
    x = RNG.standard_normal((3, 16))
    w = 1 + RNG.uniform(-0.1, 0.1, 16)
    dy = RNG.standard_normal((3, 16))
    dx = O.rmsnorm_bwd(x, w, 1e-5, dy)
    assert_fd(dx, lambda v: float(np.sum(dy * O.rmsnorm_fwd(v, w, 1e-5, rnd=identity))), x)
    y1 = O.rmsnorm_fwd(x, w, 0.0, rnd=identity)
    y2 = O.rmsnorm_fwd(3.7 * x, w, 0.0, rnd=identity)
    assert np.allclose(y1, y2, rtol=1e-13)
    c = O.rmsnorm_fwd(np.full((1, 16), -2.5), w, 0.0, rnd=identity)
    assert np.allclose(c, -w)


# ------------------------------------------------------------------ RoPE
def test_rope_is_complex_rotation():
    T, H, d, theta = 7, 3, 16, 10000.0
    x = RNG.standard_normal((T, H, d))
    pos = np.array([0, 1, 2, 3, 0, 1, 2])
    y = O.rope_apply(x, pos, theta, rnd=identity)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    freq = np.array([theta ** (-(2 * i) / d) for i in range(d // 2)])
    rot = np.exp(1j * pos[:, None, None] * freq[None, None, :])
    zr = z * rot
    assert np.allclose(y, np.concatenate([zr.real, zr.imag], -1), atol=1e-13)
    assert np.allclose(y[0], x[0]) and np.allclose(y[4], x[4])     # position 0 restarts per sequence
    back = O.rope_apply(y, pos, theta, inverse=True, rnd=identity)
    assert np.allclose(back, x, atol=1e-13)


def test_rope_relative_position():
    d, theta = 32, 500000.0
    q, k = RNG.standard_normal((1, 1, d)), RNG.standard_normal((1, 1, d))
    dots = []
    for m, n in ((5, 2), (9, 6), (103, 100)):
        qr = O.rope_apply(q, [m], theta, rnd=identity)
        kr = O.rope_apply(k, [n], theta, rnd=identity)
        dots.append(float(np.sum(qr * kr)))
    assert np.allclose(dots, dots[0], rtol=1e-10)


def test_rope_llama3_scaling_shape():
    """Llama-3.1 frequency scaling, checked by the properties that fix it: the
    ratio r = scaled / unscaled frequency is 1 where the wavelength is shorter
    than original / high_factor, 1 / factor where it is longer than
    original / low_factor, affine in x = original / wavelength in between, and
    continuous at both ends of that band."""
    factor, low, high, orig = 8.0, 1.0, 4.0, 8192.0
    d, theta = 4096, 500000.0                      # 2048 frequencies spread over the three regimes
    inv = O.rope_inv_freq(d, theta)
    r = O.rope_inv_freq(d, theta, (factor, low, high, orig)) / inv
    x = orig * inv / (2 * np.pi)                   # original / wavelength
    hi_f, lo_f, band = x > high, x < low, (x >= low) & (x <= high)
    assert hi_f.sum() > 10 and lo_f.sum() > 10 and band.sum() > 10
    assert np.all(r[hi_f] == 1.0)
    assert np.allclose(r[lo_f], 1.0 / factor, rtol=1e-15)
    xb, rb = x[band], r[band]
    slope = np.diff(rb) / np.diff(xb)
    assert np.allclose(slope, slope[0], rtol=1e-9)                       # affine in x
    assert np.isclose(rb[np.argmin(xb)] + slope[0] * (low - xb.min()), 1.0 / factor, rtol=1e-9)   # meets 1/factor at x = low
    assert np.isclose(rb[np.argmax(xb)] + slope[0] * (high - xb.max()), 1.0, rtol=1e-9)         # meets 1 at x = high
    assert np.all(np.diff(r * inv) < 0)            # frequencies stay strictly ordered
    # factor 1 changes nothing; the scaled rotation is still a rotation
    assert np.allclose(O.rope_inv_freq(128, theta, (1.0, low, high, orig)), O.rope_inv_freq(128, theta),
                       rtol=1e-15, atol=0)
    xx = RNG.standard_normal((5, 2, 128))
    y = O.rope_apply(xx, [0, 9000, 3, 40000, 7], theta, rnd=identity, scaling=(factor, low, high, orig))
    assert np.allclose(np.sum(y * y, -1), np.sum(xx * xx, -1), rtol=1e-12)
    back = O.rope_apply(y, [0, 9000, 3, 40000, 7], theta, inverse=True, rnd=identity, scaling=(factor, low, high, orig))
    assert np.allclose(back, xx, atol=1e-12)


# ------------------------------------------------------------------ attention
def _sdpa_ref(q, k, v, batch, seq):
    T, nq, d = q.shape
    grp = nq // k.shape[1]
    qt = t64(q).view(batch, seq, nq, d).transpose(1, 2)
    kt = t64(k).view(batch, seq, -1, d).transpose(1, 2).repeat_interleave(grp, dim=1)
    vt = t64(v).view(batch, seq, -1, d).transpose(1, 2).repeat_interleave(grp, dim=1)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o.transpose(1, 2).reshape(T, nq, d).numpy()


@pytest.mark.parametrize("nq,nkv", [(4, 4), (4, 2), (6, 1)])
def test_attention_matches_sdpa(nq, nkv):
    batch, seq, d = 2, 9, 8
    q = RNG.standard_normal((batch * seq, nq, d))
    k = RNG.standard_normal((batch * seq, nkv, d))
    v = RNG.standard_normal((batch * seq, nkv, d))
    o, lse = O.attention_fwd(q, k, v, batch, seq, rnd=identity)
    assert np.allclose(o, _sdpa_ref(q, k, v, batch, seq), atol=1e-12)
    # lse of the first row of every sequence is its single score
    assert np.allclose(lse[:, :, 0], np.einsum("bhd,bhd->bh",
                       q.reshape(batch, seq, nq, d)[:, 0],
                       np.repeat(k.reshape(batch, seq, nkv, d)[:, 0], nq // nkv, axis=1)) / np.sqrt(d))


def test_attention_causal_and_bwd_fd():
    batch, seq, nq, nkv, d = 2, 5, 4, 2, 4
    q = RNG.standard_normal((batch * seq, nq, d))
    k = RNG.standard_normal((batch * seq, nkv, d))
    v = RNG.standard_normal((batch * seq, nkv, d))
    do = RNG.standard_normal((batch * seq, nq, d))
    o, _ = O.attention_fwd(q, k, v, batch, seq, rnd=identity)
    k2 = k.copy(); k2[3] += 1.0                      # key at position 3 of sequence 0
    o2, _ = O.attention_fwd(q, k2, v, batch, seq, rnd=identity)
    assert np.allclose(o2[:3], o[:3]) and not np.allclose(o2[3:5], o[3:5]) and np.allclose(o2[5:], o[5:])
    dq, dk, dv = O.attention_bwd(q, k, v, do, batch, seq, rnd=identity)
    L = lambda qq, kk, vv: float(np.sum(do * O.attention_fwd(qq, kk, vv, batch, seq, rnd=identity)[0]))
    assert_fd(dq, lambda z: L(z, k, v), q)
    assert_fd(dk, lambda z: L(q, z, v), k)
    assert_fd(dv, lambda z: L(q, k, z), v)


# ------------------------------------------------------------------ SwiGLU
def test_swiglu_matches_torch_and_fd():
    g, u, da = (RNG.standard_normal((4, 6)) * 3 for _ in range(3))
    a = O.swiglu_fwd(g, u, rnd=identity)
    assert np.allclose(a, (F.silu(t64(g)) * t64(u)).numpy(), atol=1e-14)
    dg, du = O.swiglu_bwd(g, u, da, rnd=identity)
    assert_fd(dg, lambda z: float(np.sum(da * O.swiglu_fwd(z, u, rnd=identity))), g)
    assert_fd(du, lambda z: float(np.sum(da * O.swiglu_fwd(g, z, rnd=identity))), u)


# ------------------------------------------------------------------ decoder layer
def tiny_layer_params(shape=TINY_LAYER, seed=3):
    rng = np.random.default_rng(seed)
    w = {p: rng.standard_normal((fout, fin)) * 0.1 for p, (fin, fout) in PROJ_IN_OUT(shape).items()}
    w["norm1"] = 1 + rng.uniform(-0.1, 0.1, shape.hidden)
    w["norm2"] = 1 + rng.uniform(-0.1, 0.1, shape.hidden)
    lora = {}
    for p, (fin, fout) in PROJ_IN_OUT(shape).items():
        lora["A_" + p] = rng.uniform(-0.3, 0.3, (shape.lora_r, fin))
        lora["B_" + p] = rng.standard_normal((fout, shape.lora_r)) * 0.1
    return w, lora


def _torch_layer(x, w, lora, shape, batch, seq):
    """Independent composition from torch library ops (merged LoRA weights, SDPA,
    F.linear's own bias)."""
    s = shape.lora_scale
    W = {p: t64(w[p]) + s * (t64(lora["B_" + p]) @ t64(lora["A_" + p])) for p in PROJ_IN_OUT(shape)}
    xt = t64(x)
    n1 = F.rms_norm(xt, (shape.hidden,), t64(w["norm1"]), eps=shape.rms_eps)
    T, d = x.shape[0], shape.head_dim
    q, k, v = (F.linear(n1, W[p], t64(w[p + "_bias"]) if p + "_bias" in w else None).numpy()
               for p in ("q", "k", "v"))
    pos = np.tile(np.arange(seq), batch)

    def rot(a, nh):
        a = a.reshape(T, nh, d)
        z = a[..., : d // 2] + 1j * a[..., d // 2:]
        fr = shape.rope_theta ** (-(2 * np.arange(d // 2)) / d)
        z = z * np.exp(1j * pos[:, None, None] * fr[None, None, :])
        return np.concatenate([z.real, z.imag], -1)
    o = _sdpa_ref(rot(q, shape.n_q), rot(k, shape.n_kv), v.reshape(T, shape.n_kv, d), batch, seq)
    h1 = xt + F.linear(t64(o.reshape(T, -1)), W["o"])
    n2 = F.rms_norm(h1, (shape.hidden,), t64(w["norm2"]), eps=shape.rms_eps)
    a = F.silu(F.linear(n2, W["gate"])) * F.linear(n2, W["up"])
    return (h1 + F.linear(a, W["down"])).numpy()


def test_decoder_layer_fwd_matches_torch_composition():
    shape, batch, seq = TINY_LAYER, 2, 8
    w, lora = tiny_layer_params()
    x = RNG.standard_normal((batch * seq, shape.hidden))
    out, _ = O.decoder_layer_fwd(x, w, lora, shape, batch, seq, rnd=identity)
    assert np.allclose(out, _torch_layer(x, w, lora, shape, batch, seq), atol=1e-11)


def test_decoder_layer_qkv_bias_matches_torch_and_shifts_v():
    """q/k/v bias: the layer equals torch's composition with F.linear's bias, and
    a v bias alone moves the attention output by exactly that bias (softmax rows
    sum to one)."""
    import dataclasses
    shape, batch, seq = dataclasses.replace(TINY_LAYER, qkv_bias=True), 2, 8
    w, lora = tiny_layer_params()
    rng = np.random.default_rng(5)
    for p, n in (("q", shape.q_dim), ("k", shape.kv_dim), ("v", shape.kv_dim)):
        w[p + "_bias"] = rng.standard_normal(n) * 0.5
    x = RNG.standard_normal((batch * seq, shape.hidden))
    out, c = O.decoder_layer_fwd(x, w, lora, shape, batch, seq, rnd=identity)
    assert np.allclose(out, _torch_layer(x, w, lora, shape, batch, seq), atol=1e-11)
    w0 = dict(w); w0["v_bias"] = np.zeros(shape.kv_dim)
    _, c0 = O.decoder_layer_fwd(x, w0, lora, shape, batch, seq, rnd=identity)
    grp = shape.n_q // shape.n_kv
    shift = np.repeat(w["v_bias"].reshape(shape.n_kv, shape.head_dim), grp, axis=0).reshape(-1)
    assert np.allclose(c["attn"] - c0["attn"], shift[None, :], atol=1e-12)


def test_decoder_layer_bwd_finite_differences_with_bias_and_scaling():
    """The backward stays the gradient of the forward with q/k/v bias and
    Llama-3.1 RoPE scaling switched on (positions past the original context)."""
    import dataclasses
    shape = dataclasses.replace(TINY_LAYER, qkv_bias=True, rope_scaling=(8.0, 1.0, 4.0, 64.0))
    batch, seq = 1, 8
    w, lora = tiny_layer_params()
    rng = np.random.default_rng(13)
    for p, n in (("q", shape.q_dim), ("k", shape.kv_dim), ("v", shape.kv_dim)):
        w[p + "_bias"] = rng.standard_normal(n) * 0.5
    x = rng.standard_normal((batch * seq, shape.hidden))
    dout = rng.standard_normal((batch * seq, shape.hidden))
    dx, gr = O.decoder_layer_bwd(x, dout, w, lora, shape, batch, seq, rnd=identity)

    def L(xx=x, ll=lora):
        return float(np.sum(dout * O.decoder_layer_fwd(xx, w, ll, shape, batch, seq, rnd=identity)[0]))
    assert_fd(dx, lambda v: L(xx=v), x, n=8, rtol=1e-5, atol=1e-8)
    for key in ("A_q", "B_k", "B_v"):
        def Lk(v, key=key):
            ll = dict(lora); ll[key] = v
            return L(ll=ll)
        assert_fd(gr[key], Lk, lora[key], n=4, rtol=1e-5, atol=1e-8)


def test_decoder_layer_bwd_finite_differences():
    shape, batch, seq = TINY_LAYER, 1, 8
    w, lora = tiny_layer_params()
    rng = np.random.default_rng(11)
    x = rng.standard_normal((batch * seq, shape.hidden))
    dout = rng.standard_normal((batch * seq, shape.hidden))
    dx, gr = O.decoder_layer_bwd(x, dout, w, lora, shape, batch, seq, rnd=identity)

    def L(xx=x, ll=lora):
        return float(np.sum(dout * O.decoder_layer_fwd(xx, w, ll, shape, batch, seq, rnd=identity)[0]))
    assert_fd(dx, lambda v: L(xx=v), x, n=8, rtol=1e-5, atol=1e-8)
    for key in ("A_q", "B_k", "A_v", "B_o", "A_gate", "B_up", "A_down", "B_down"):
        def Lk(v, key=key):
            ll = dict(lora); ll[key] = v
            return L(ll=ll)
        assert_fd(gr[key], Lk, lora[key], n=4, rtol=1e-5, atol=1e-8)


def test_decoder_layer_zero_b_gives_zero_da():
    shape, batch, seq = TINY_LAYER, 1, 8
    w, lora = tiny_layer_params()
    for p in PROJ_IN_OUT(shape):
        lora["B_" + p] = np.zeros_like(lora["B_" + p])
    x = RNG.standard_normal((seq, shape.hidden))
    dout = RNG.standard_normal((seq, shape.hidden))
    _, gr = O.decoder_layer_bwd(x, dout, w, lora, shape, batch, seq, rnd=identity)
    for p in PROJ_IN_OUT(shape):
        assert np.all(gr["A_" + p] == 0) and np.any(gr["B_" + p] != 0)


# ------------------------------------------------------------------ cross-entropy
def test_ce_matches_torch():
    T, H, V = 12, 16, 50
    h = RNG.standard_normal((T, H))
    W = RNG.standard_normal((V, H)) * 0.3
    labels = RNG.integers(0, V, T)
    labels[[3, 7]] = -100
    loss, lse, nv = O.ce_loss_fwd(h, W, labels)
    ht = t64(h).requires_grad_(True)
    ref = F.cross_entropy(ht @ t64(W).T, torch.from_numpy(labels), ignore_index=-100)
    assert nv == 10 and abs(loss - ref.item()) < 1e-12
    assert np.allclose(lse, torch.logsumexp(t64(h) @ t64(W).T, dim=1).numpy())
    ref.backward()
    dh = O.ce_loss_bwd(h, W, labels, rnd=identity)
    assert np.allclose(dh, ht.grad.numpy(), atol=1e-13)
    assert np.all(dh[[3, 7]] == 0)
    dh2 = O.ce_loss_bwd(h, W, labels, grad_scale=0.25, rnd=identity)
    assert np.allclose(dh2, 0.25 * dh)


def test_ce_token_logprobs_match_torch_log_softmax():
    """logp = log_softmax(z)[label] from torch, 0 where ignored; W = 0 gives
    -ln V; over every possible label the probabilities sum to one; the
    per-sequence score is the sum of its tokens."""
    from oracle.ce import ce_token_logprobs, sequence_logprobs
    T, H, V = 12, 16, 50
    h = RNG.standard_normal((T, H))
    W = RNG.standard_normal((V, H)) * 0.3
    labels = RNG.integers(0, V, T)
    labels[[3, 7]] = -100
    lp = ce_token_logprobs(h, W, labels)
    ref = torch.log_softmax(t64(h) @ t64(W).T, dim=1).numpy()
    ok = labels != -100
    assert np.allclose(lp[ok], ref[np.nonzero(ok)[0], labels[ok]], atol=1e-13) and np.all(lp[~ok] == 0)
    assert np.allclose(ce_token_logprobs(h, np.zeros((V, H)), labels)[ok], -np.log(V), atol=1e-13)
    every = np.array([ce_token_logprobs(h[:1], W, [v])[0] for v in range(V)])
    assert abs(np.exp(every).sum() - 1.0) < 1e-12
    assert np.allclose(sequence_logprobs(lp, 3, 4), [lp[0:4].sum(), lp[4:8].sum(), lp[8:12].sum()])
    loss, _, nv = O.ce_loss_fwd(h, W, labels)
    assert abs(loss + lp.sum() / nv) < 1e-12          # the training loss is minus their mean


def test_adapter_off_layer_equals_zero_b_and_torch():
    """With the adapters off the layer is the base alone: bit for bit the layer
    with B = 0 (in bf16 mode, where t B^T = 0 exactly), and torch's
    composition of the plain weights."""
    shape, batch, seq = TINY_LAYER, 2, 8
    w, lora = tiny_layer_params()
    x = RNG.standard_normal((batch * seq, shape.hidden))
    off, c = O.decoder_layer_fwd(x, w, None, shape, batch, seq)
    lora0 = {k: (np.zeros_like(v) if k.startswith("B_") else v) for k, v in lora.items()}
    zero_b, _ = O.decoder_layer_fwd(x, w, lora0, shape, batch, seq)
    assert np.array_equal(off, zero_b) and c["t_q"] is None
    exact, _ = O.decoder_layer_fwd(x, w, None, shape, batch, seq, rnd=identity)
    assert np.allclose(exact, _torch_layer(x, w, lora0, shape, batch, seq), atol=1e-11)
    # and it is not the adapted layer
    assert not np.allclose(exact, O.decoder_layer_fwd(x, w, lora, shape, batch, seq, rnd=identity)[0])


def test_ce_zero_weights_closed_form():
    T, H, V = 5, 8, 37
    h = RNG.standard_normal((T, H))
    loss, lse, _ = O.ce_loss_fwd(h, np.zeros((V, H)), RNG.integers(0, V, T))
    assert abs(loss - math.log(V)) < 1e-14 and np.allclose(lse, math.log(V))
    assert np.all(O.ce_loss_bwd(h, np.zeros((V, H)), RNG.integers(0, V, T)) == 0)


def test_ce_bwd_fd():
    T, H, V = 4, 6, 11
    h = RNG.standard_normal((T, H))
    W = RNG.standard_normal((V, H))
    labels = np.array([1, 5, -100, 10])
    dh = O.ce_loss_bwd(h, W, labels, rnd=identity)
    assert_fd(dh, lambda v: O.ce_loss_fwd(v, W, labels)[0], h)


# ------------------------------------------------------------------ AdamW
def test_adamw_matches_torch_and_first_step():
    p0 = RNG.standard_normal(10)
    pt = t64(p0).clone().requires_grad_(True)
    opt = torch.optim.AdamW([pt], lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    p, m, v = p0.copy(), np.zeros(10), np.zeros(10)
    for step in range(1, 5):
        g = RNG.standard_normal(10)
        pt.grad = t64(g)
        opt.step()
        p_prev = p
        p, m, v = O.adamw_step(p, g, m, v, step, lr=2e-4, wd=0.01)
        if step == 1:
            # p1 = p0 (1 - lr wd) - lr g / (|g| + eps)
            assert np.allclose(p, p_prev * (1 - 2e-6) - 2e-4 * g / (np.abs(g) + 1e-8), rtol=1e-12, atol=1e-15)
    assert np.allclose(p, pt.detach().numpy(), rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------ whole model
def test_model_grad_reaches_layer0_fd():
    """The gradient of the mean loss with respect to a layer-0 adapter equals its
    finite difference (a severed path upstream would make it zero or wrong)."""
    from oracle.model import model_step
    shape, batch, seq, V = TINY_LAYER, 1, 6, 23
    rng = np.random.default_rng(5)
    layers = [tiny_layer_params(seed=s) for s in (21, 22)]
    emb = rng.standard_normal((V, shape.hidden)) * 0.5
    fn = np.ones(shape.hidden)
    ids = [rng.integers(0, V, seq), rng.integers(0, V, seq)]
    loss, grads, _ = model_step(ids, emb, fn, None, layers, shape, batch, seq, rnd=identity)
    key = "A_q"
    a0 = layers[0][1][key]

    def L(v):
        ll = [(layers[0][0], {**layers[0][1], key: v}), layers[1]]
        return model_step(ids, emb, fn, None, ll, shape, batch, seq, rnd=identity)[0]
    assert_fd(grads[0][key], L, a0, n=4, rtol=1e-5, atol=1e-9)
    assert np.any(grads[0][key] != 0)


def test_reference_logprobs_agree_with_the_training_loss_at_b_zero():
    """The adapter-off forward scores each token; with B = 0 the adapted
    model computes the same forward, so its training loss is minus the mean
    reference log-probability, and each sequence score is the sum of its own
    tokens' log-probabilities."""
    from oracle.model import model_fwd_bwd, reference_logprobs
    shape, batch, seq, V = TINY_LAYER, 2, 6, 23
    rng = np.random.default_rng(9)
    layers = [tiny_layer_params(seed=s) for s in (31, 32)]
    layers0 = [(w, {k: (np.zeros_like(v) if k.startswith("B_") else v) for k, v in lo.items()}) for w, lo in layers]
    emb = rng.standard_normal((V, shape.hidden)) * 0.5
    fn = 1 + rng.uniform(-0.1, 0.1, shape.hidden)
    ids = rng.integers(0, V, batch * seq)
    lp, slp = reference_logprobs(ids, emb, fn, None, [w for w, _ in layers], shape, batch, seq)
    r = model_fwd_bwd(ids, emb, fn, None, layers0, shape, batch, seq)
    assert r["n_valid"] == batch * (seq - 1)
    assert abs(r["loss"] + lp.sum() / r["n_valid"]) < 1e-12
    assert np.all(lp.reshape(batch, seq)[:, -1] == 0) and np.all(lp.reshape(batch, seq)[:, :-1] < 0)
    assert np.allclose(slp, lp.reshape(batch, seq).sum(1))


# ------------------------------------------------------------------ model composition
def _torch_model_loss(ids, emb, fn, lm_head, layers, shape, batch, seq):
    """Loss, per-token LSE and adapter gradients of a whole model built from torch
    float64 library ops with autograd, independent of the oracle: F.embedding,
    merged LoRA weights in F.linear, a complex rotation for RoPE, SDPA with
    repeated kv heads, F.rms_norm, and F.cross_entropy on logits[:, :-1] against
    ids[:, 1:] (each sequence predicts its own next token). The head is the
    embedding table when lm_head is None."""
    s, d, H = shape.lora_scale, shape.head_dim, shape.hidden
    T = batch * seq
    pos = torch.from_numpy(np.tile(np.arange(seq), batch).astype(np.float64))
    fr = torch.from_numpy(shape.rope_theta ** (-(2 * np.arange(d // 2)) / d))
    phase = torch.exp(1j * pos[:, None, None] * fr[None, None, :])
    params = []
    h = F.embedding(torch.from_numpy(np.asarray(ids, np.int64)), t64(emb))
    for w, lora in layers:
        A = {p: t64(lora["A_" + p]).requires_grad_(True) for p in PROJ_IN_OUT(shape)}
        B = {p: t64(lora["B_" + p]).requires_grad_(True) for p in PROJ_IN_OUT(shape)}
        params.append((A, B))
        W = {p: t64(w[p]) + s * (B[p] @ A[p]) for p in PROJ_IN_OUT(shape)}
        n1 = F.rms_norm(h, (H,), t64(w["norm1"]), eps=shape.rms_eps)

        def rot(a, nh):
            a = a.reshape(T, nh, d)
            z = torch.complex(a[..., : d // 2], a[..., d // 2:]) * phase
            return torch.cat([z.real, z.imag], -1)
        grp = shape.n_q // shape.n_kv
        q = rot(F.linear(n1, W["q"]), shape.n_q).view(batch, seq, shape.n_q, d).transpose(1, 2)
        k = rot(F.linear(n1, W["k"]), shape.n_kv).view(batch, seq, shape.n_kv, d).transpose(1, 2)
        v = F.linear(n1, W["v"]).view(batch, seq, shape.n_kv, d).transpose(1, 2)
        o = F.scaled_dot_product_attention(q, k.repeat_interleave(grp, 1), v.repeat_interleave(grp, 1),
                                           is_causal=True)
        h = h + F.linear(o.transpose(1, 2).reshape(T, -1), W["o"])
        n2 = F.rms_norm(h, (H,), t64(w["norm2"]), eps=shape.rms_eps)
        h = h + F.linear(F.silu(F.linear(n2, W["gate"])) * F.linear(n2, W["up"]), W["down"])
    hn = F.rms_norm(h, (H,), t64(fn), eps=shape.rms_eps)
    logits = hn @ t64(emb if lm_head is None else lm_head).T
    V = logits.shape[-1]
    tgt = torch.from_numpy(np.asarray(ids, np.int64)).view(batch, seq)[:, 1:].reshape(-1)
    loss = F.cross_entropy(logits.view(batch, seq, V)[:, :-1].reshape(-1, V), tgt)
    loss.backward()
    grads = [{**{"A_" + p: A[p].grad.numpy() for p in A}, **{"B_" + p: B[p].grad.numpy() for p in B}}
             for A, B in params]
    return float(loss), torch.logsumexp(logits, -1).detach().numpy(), grads


@pytest.mark.parametrize("tied", [True, False])
def test_model_composition_matches_torch(tied):
    """The oracle's microbatch (embedding gather, layers, final RMSNorm, head,
    shifted-label cross-entropy) and its backward through every layer equal a
    torch autograd composition: loss and LSE to 1e-12, adapter gradients to 1e-9.
    Two sequences, so a label shift across the sequence boundary (or no shift,
    or a reversed one) fails; distinct emb and lm_head, so a swapped head fails."""
    from oracle.model import model_fwd_bwd
    shape, batch, seq, V = TINY_LAYER, 2, 7, 29
    rng = np.random.default_rng(11 + tied)
    layers = [tiny_layer_params(seed=s) for s in (41, 42)]
    emb = rng.standard_normal((V, shape.hidden)) * 0.5
    lm = None if tied else rng.standard_normal((V, shape.hidden)) * 0.5
    fn = 1 + rng.uniform(-0.1, 0.1, shape.hidden)
    ids = rng.integers(0, V, batch * seq)
    r = model_fwd_bwd(ids, emb, fn, lm, layers, shape, batch, seq, rnd=identity)
    loss, lse, grads = _torch_model_loss(ids, emb, fn, lm, layers, shape, batch, seq)
    assert r["n_valid"] == batch * (seq - 1)
    assert abs(r["loss"] - loss) <= 1e-12 * abs(loss), (r["loss"], loss)
    assert np.allclose(r["lse"], lse, rtol=0, atol=1e-12)
    for li in range(len(layers)):
        for k, g in grads[li].items():
            assert np.allclose(r["grads"][li][k], g, rtol=1e-9, atol=1e-12), (li, k)
            assert np.any(g != 0), (li, k)
