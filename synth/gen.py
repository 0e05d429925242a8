"""Seeded tensor generators (data preparation only, no method arithmetic)."""
import numpy as np

from .configs import TENSOR_IDS, HEAD_LAYER_ID, LORA_PROJ, PROJ_IN_OUT, LayerShape


def stream(wid: int, layer_id: int, tensor_id: int, salt: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for one tensor of one layer of one workload."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, layer_id, tensor_id, salt])))


def _to_bf16_values(f32: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 (ties to even) of finite float32 input, as float32 values."""
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def as_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Raw 16-bit patterns of float32 values that are exact bfloat16 values."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    u = v.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not exactly representable in bfloat16")
    return (u >> 16).astype(np.uint16)


def normal_bf16(shape, std, wid, layer_id, tensor_id, salt=0):
    g = stream(wid, layer_id, tensor_id, salt)
    return _to_bf16_values(g.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def uniform_bf16(shape, lo, hi, wid, layer_id, tensor_id, salt=0):
    g = stream(wid, layer_id, tensor_id, salt)
    return _to_bf16_values(g.uniform(lo, hi, size=shape).astype(np.float32))


def norm_weight_bf16(n, wid, layer_id, tensor_id, ones: bool):
    """RMSNorm weight: all ones (benches) or 1 + U(-0.1, 0.1) (tests)."""
    if ones:
        return np.ones(n, np.float32)
    g = stream(wid, layer_id, tensor_id)
    return _to_bf16_values((1.0 + g.uniform(-0.1, 0.1, size=n)).astype(np.float32))


def token_ids(n, vocab, wid, salt=0):
    g = stream(wid, HEAD_LAYER_ID, TENSOR_IDS["tokens"], salt)
    return g.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def activation(shape, wid, name, salt=0, std=1.0):
    """x or dy ~ N(0, std) as bfloat16 values."""
    return normal_bf16(shape, std, wid, 0, TENSOR_IDS[name], salt)


def layer_weights(shape: LayerShape, wid: int, layer_id: int, w_std=0.02, ones_norm=False, bias_std=0.1):
    """Frozen base weights of one decoder layer, unquantised bf16 values [out x in]
    (plus 'q_bias', 'k_bias', 'v_bias' ~ N(0, bias_std) when the shape has them)."""
    out = {}
    for p, (fin, fout) in PROJ_IN_OUT(shape).items():
        out[p] = normal_bf16((fout, fin), w_std, wid, layer_id, TENSOR_IDS[p])
    out["norm1"] = norm_weight_bf16(shape.hidden, wid, layer_id, TENSOR_IDS["norm1"], ones_norm)
    out["norm2"] = norm_weight_bf16(shape.hidden, wid, layer_id, TENSOR_IDS["norm2"], ones_norm)
    if getattr(shape, "qkv_bias", False):
        for p, n in (("q", shape.q_dim), ("k", shape.kv_dim), ("v", shape.kv_dim)):
            out[p + "_bias"] = normal_bf16((n,), bias_std, wid, layer_id, TENSOR_IDS[p + "_bias"])
    return out


def layer_lora(shape: LayerShape, wid: int, layer_id: int, b_std=0.01, b_zero=False):
    """LoRA parameters: A [r x in] ~ U(+-1/sqrt(in)), B [out x r] ~ N(0, b_std) (or zeros)."""
    r = shape.lora_r
    out = {}
    for p, (fin, fout) in PROJ_IN_OUT(shape).items():
        lim = 1.0 / np.sqrt(fin)
        out["A_" + p] = uniform_bf16((r, fin), -lim, lim, wid, layer_id, TENSOR_IDS["A_" + p])
        if b_zero:
            out["B_" + p] = np.zeros((fout, r), np.float32)
        else:
            out["B_" + p] = normal_bf16((fout, r), b_std, wid, layer_id, TENSOR_IDS["B_" + p])
    return out


def model_head(hidden, vocab, tied, wid, std=0.02, ones_norm=True):
    """Embedding table [V x H], final norm weight [H], lm_head [V x H] (None when tied)."""
    emb = normal_bf16((vocab, hidden), std, wid, HEAD_LAYER_ID, TENSOR_IDS["embed"])
    fn = norm_weight_bf16(hidden, wid, HEAD_LAYER_ID, TENSOR_IDS["final_norm"], ones_norm)
    lm = None if tied else normal_bf16((vocab, hidden), std, wid, HEAD_LAYER_ID, TENSOR_IDS["lm_head"])
    return emb, fn, lm


__all__ = ["stream", "normal_bf16", "uniform_bf16", "norm_weight_bf16", "token_ids",
           "as_bf16_bits", "layer_weights", "layer_lora", "model_head", "activation",
           "LORA_PROJ"]
