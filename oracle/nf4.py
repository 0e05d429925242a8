"""NF4: 4-bit NormalFloat with blockwise absmax scaling (block 64, float32 absmax).

The pages name NF4 as the format of the frozen 8B base ("Exact Layer
Streaming ...", abstract; "Soup CLI ...", "Key Takeaways"). Its definition is
QLoRA's NormalFloat (Dettmers et al. 2023, section 3): the code values are
quantiles of the standard normal distribution, split so that zero is exactly
representable, scaled to [-1, 1].

Readings taken here (the pages are silent on all of them):
  * offset delta = ((1 - 1/30) + (1 - 1/32)) / 2 = 929/960, evaluated in float64;
  * 8 positive values: Phi^-1 at 8 evenly spaced probabilities from delta down
    to (but excluding) 1/2 (9-point grid, last point dropped); 7 negative values:
    the same with an 8-point grid, negated; plus an exact 0; every value is
    divided by the largest (Phi^-1(delta)) in float64 and rounded once to float32;
  * quantisation: w is the bf16 weight read as float32; absmax per block of 64
    consecutive row-major elements; n = w / absmax (float32, IEEE division;
    n = 0 when absmax = 0); code = number of float32 midpoints
    m_i = (c_i + c_{i+1}) / 2 with n > m_i (nearest code, ties to the lower index);
  * packing: element 2j in the high nibble of byte j, element 2j+1 in the low nibble;
  * dequantisation: w' = bf16(float32(c[code]) * absmax), one float32 multiply.
"""
from statistics import NormalDist

import numpy as np

from .bf16 import round_bf16

BLOCK = 64


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 code values, ascending, float32."""
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    nd = NormalDist()
    pos = [nd.inv_cdf(p) for p in np.linspace(delta, 0.5, 9)[:-1]]
    neg = [-nd.inv_cdf(p) for p in np.linspace(delta, 0.5, 8)[:-1]]
    vals = sorted(pos + neg + [0.0])
    top = max(vals)
    return np.array([v / top for v in vals], dtype=np.float64).astype(np.float32)


def _midpoints(cb: np.ndarray) -> np.ndarray:
    cb = cb.astype(np.float32)
    return ((cb[:-1] + cb[1:]) * np.float32(0.5)).astype(np.float32)


def nf4_quantize(w: np.ndarray):
    """Quantise w [rows x cols] (cols % 64 == 0) -> (codes uint8 [rows x cols/2], absmax float32 [rows x cols/64])."""
    w = np.asarray(w)
    rows, cols = w.shape
    if cols % BLOCK:
        raise ValueError("in-features must be a multiple of 64")
    f = w.astype(np.float32).reshape(-1, BLOCK)
    absmax = np.max(np.abs(f), axis=1).astype(np.float32)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    n = (f / safe[:, None]).astype(np.float32)
    n[absmax == 0] = np.float32(0.0)
    mids = _midpoints(nf4_codebook())
    code = np.sum(n[..., None] > mids[None, None, :], axis=-1).astype(np.uint8)
    code = code.reshape(rows, cols)
    packed = ((code[:, 0::2] << 4) | code[:, 1::2]).astype(np.uint8)
    return packed, absmax.reshape(rows, cols // BLOCK)


def nf4_unpack(packed: np.ndarray) -> np.ndarray:
    """Codes uint8 [rows x cols] from packed bytes [rows x cols/2]."""
    rows, half = packed.shape
    code = np.empty((rows, 2 * half), np.uint8)
    code[:, 0::2] = packed >> 4
    code[:, 1::2] = packed & 0xF
    return code


def nf4_dequant(packed: np.ndarray, absmax: np.ndarray, rnd=round_bf16) -> np.ndarray:
    """w' = rnd(float32(c[code]) * absmax) as float64 [rows x cols]."""
    code = nf4_unpack(packed)
    rows, cols = code.shape
    cb = nf4_codebook()
    c = cb[code].reshape(-1, BLOCK)
    prod = (c * absmax.reshape(-1)[:, None].astype(np.float32)).astype(np.float32)
    return rnd(prod.astype(np.float64)).reshape(rows, cols)


# ---------------------------------------------------------------- double quantisation
# The pages' sizes ("Soup: ...", section "Layer Streaming: The Mechanism Behind
# the 4 GB Claim": a 3.60 GB base store over 32 layers and two 113 MB buffers
# for Llama-3.1-8B) equal 4-bit codes plus one 8-bit absmax code per 64 weights
# plus one float32 constant per 256 absmax values. The pages fix only those byte
# counts, not the 8-bit map, so the map below is this build's own reading, the
# plainest linear one that fits the sizes. (It is not QLoRA's double
# quantization, which maps the mean-centred constants with 8-bit floats; that
# scheme has the same byte count.)
#   * s = float32(max of the 256 absmax values / 255) (float32 division);
#   * q = round-half-even(absmax / s) (float32 division), clamped to [0, 255];
#     q = 0 when s = 0;
#   * absmax' = float32(q) * s (one float32 multiply); absmax values are
#     flattened in row-major order and the last block may be short;
#   * the 4-bit codes are those of nf4_quantize (chosen with the exact absmax);
#     dequantisation uses absmax': w' = bf16(float32(c[code]) * absmax').
DQ_BLOCK = 256


def nf4dq_quantize_absmax(absmax: np.ndarray):
    """float32 absmax [rows x nb] -> (q uint8 [rows x nb], scale float32 [ceil(rows*nb/256)])."""
    a = np.asarray(absmax, np.float32).reshape(-1)
    nblk = (a.size + DQ_BLOCK - 1) // DQ_BLOCK
    scale = np.empty(nblk, np.float32)
    q = np.empty(a.size, np.uint8)
    for b in range(nblk):
        blk = a[b * DQ_BLOCK:(b + 1) * DQ_BLOCK]
        s = np.float32(np.max(blk) / np.float32(255.0))
        scale[b] = s
        if s > 0:
            r = np.rint((blk / s).astype(np.float32))
            q[b * DQ_BLOCK:(b + 1) * DQ_BLOCK] = np.clip(r, 0, 255).astype(np.uint8)
        else:
            q[b * DQ_BLOCK:(b + 1) * DQ_BLOCK] = 0
    return q.reshape(np.shape(absmax)), scale


def nf4dq_absmax(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """absmax' = float32(q) * s of its 256-block, same shape as q."""
    qf = np.asarray(q, np.uint8).reshape(-1).astype(np.float32)
    s = np.repeat(np.asarray(scale, np.float32), DQ_BLOCK)[:qf.size]
    return (qf * s).astype(np.float32).reshape(np.shape(q))


def nf4dq_quantize(w: np.ndarray):
    """w [rows x cols] -> (codes uint8 [rows x cols/2], q uint8 [rows x cols/64], scale float32)."""
    packed, absmax = nf4_quantize(w)
    q, scale = nf4dq_quantize_absmax(absmax)
    return packed, q, scale


def nf4dq_dequant(packed: np.ndarray, q: np.ndarray, scale: np.ndarray, rnd=round_bf16) -> np.ndarray:
    """w' = rnd(float32(c[code]) * absmax') as float64 [rows x cols]."""
    return nf4_dequant(packed, nf4dq_absmax(q, scale), rnd)


def nf4dq_layer_bytes(hidden, n_q, n_kv, head_dim, inter):
    """Bytes of one decoder layer stored this way: 4-bit codes, 8-bit absmax,
    float32 block constants for the seven projections, and the two bf16 norm
    weights (no alignment padding)."""
    q, kv = n_q * head_dim, n_kv * head_dim
    mats = [(q, hidden), (kv, hidden), (kv, hidden), (hidden, q), (inter, hidden), (inter, hidden), (hidden, inter)]
    total = 2 * 2 * hidden
    for n, k in mats:
        nb = n * k // BLOCK
        total += n * k // 2 + nb + 4 * ((nb + DQ_BLOCK - 1) // DQ_BLOCK)
    return total


def nf4dq_quantize_fused(mats):
    """Double quantization of several matrices with the same column count that
    are stored one under another as one fused matrix (the q, k and v weights;
    gate and up): the 4-bit codes and absmax are those of each matrix alone,
    and the absmax values of the stacked matrix, flattened row-major, are cut
    into blocks of 256 as one vector, so a block may straddle two matrices.
    This is the same as double-quantizing each matrix alone whenever every
    matrix holds a multiple of 256 absmax values (any rows x cols with both
    multiples of 128). Returns the dequantised matrices (float64, as
    nf4dq_dequant)."""
    stacked = np.concatenate([np.asarray(m, np.float64) for m in mats], axis=0)
    packed, q, scale = nf4dq_quantize(stacked)
    w = nf4dq_dequant(packed, q, scale)
    out, r = [], 0
    for m in mats:
        out.append(w[r:r + m.shape[0]])
        r += m.shape[0]
    return out
