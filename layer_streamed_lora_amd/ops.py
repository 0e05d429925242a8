"""Python binding of the C ABI, one function per entry point, same names.

Argument marshalling only: torch tensors provide device memory and streams;
every computation runs in the HIP library. There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
import ctypes as C

import torch

from . import _abi

_LIB = None


class LslError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {_abi.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib():
    global _LIB
    if _LIB is None:
        _LIB = _abi.load()
    return _LIB


def _check(fn, st):
    if st != _abi.LSL_OK:
        raise LslError(fn, st, lib().lsl_last_error().decode())


def _p(t):
    return None if t is None else t.data_ptr()


def _s(stream=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _need(t, dtype, name):
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype}, got {t.dtype} contiguous={t.is_contiguous()}")


def abi_version():
    return lib().lsl_abi_version()


def device_info(device=0):
    p = _abi.DeviceProps()
    _check("lsl_device_info", lib().lsl_device_info(device, C.byref(p)))
    return {"cu_count": p.cu_count, "clock_khz": p.clock_khz, "mem_clock_khz": p.mem_clock_khz,
            "mem_bus_bits": p.mem_bus_bits, "hbm_bytes": p.hbm_bytes, "lds_bytes_per_cu": p.lds_bytes_per_cu,
            "arch": p.arch.decode()}


# ------------------------------------------------------------------ NF4
def nf4_codebook():
    out = (C.c_float * 16)()
    _check("lsl_nf4_codebook", lib().lsl_nf4_codebook(out))
    return list(out)


def nf4_quantize(w, stream=None):
    _need(w, torch.bfloat16, "w")
    rows, cols = w.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=w.device)
    absmax = torch.empty((rows, cols // 64), dtype=torch.float32, device=w.device)
    _check("lsl_nf4_quantize", lib().lsl_nf4_quantize(_p(w), rows, cols, _p(codes), _p(absmax), _s(stream)))
    return codes, absmax


def nf4_dequant(codes, absmax, stream=None):
    rows, half = codes.shape
    w = torch.empty((rows, 2 * half), dtype=torch.bfloat16, device=codes.device)
    _check("lsl_nf4_dequant", lib().lsl_nf4_dequant(_p(codes), _p(absmax), rows, 2 * half, _p(w), _s(stream)))
    return w


def nf4dq_quantize_absmax(absmax, stream=None):
    """float32 absmax (any shape, flattened row-major) -> (uint8 codes, float32
    per-256-block constants)."""
    _need(absmax, torch.float32, "absmax")
    n = absmax.numel()
    q = torch.empty(absmax.shape, dtype=torch.uint8, device=absmax.device)
    scale = torch.empty(((n + 255) // 256,), dtype=torch.float32, device=absmax.device)
    _check("lsl_nf4dq_quantize_absmax",
           lib().lsl_nf4dq_quantize_absmax(_p(absmax), n, _p(q), _p(scale), _s(stream)))
    return q, scale


def nf4dq_dequant(codes, q, scale, stream=None):
    rows, half = codes.shape
    w = torch.empty((rows, 2 * half), dtype=torch.bfloat16, device=codes.device)
    _check("lsl_nf4dq_dequant",
           lib().lsl_nf4dq_dequant(_p(codes), _p(q), _p(scale), rows, 2 * half, _p(w), _s(stream)))
    return w


# ------------------------------------------------------------------ weights
class FrozenWeight:
    """A frozen [n_out x k_in] weight: NF4 (codes, absmax), NF4 with
    double-quantized absmax (codes, absmax_q, absmax_scale) or bf16."""

    def __init__(self, n_out, k_in, codes=None, absmax=None, bf16=None, absmax_q=None, absmax_scale=None,
                 bias=None):
        self.n_out, self.k_in = n_out, k_in
        self.codes, self.absmax, self.bf16 = codes, absmax, bf16
        self.absmax_q, self.absmax_scale, self.bias = absmax_q, absmax_scale, bias
        if bf16 is not None:
            self.fmt = _abi.WFMT_BF16
        elif absmax_q is not None:
            self.fmt = _abi.WFMT_NF4DQ
        else:
            self.fmt = _abi.WFMT_NF4
        self.struct = _abi.Weight(self.fmt, 0, n_out, k_in, _p(codes), _p(absmax), _p(bf16),
                                  _p(absmax_q), _p(absmax_scale), _p(bias))

    def with_bias(self, bias):
        """The same weight with a frozen bf16 bias [n_out] added to its forward output."""
        return FrozenWeight(self.n_out, self.k_in, self.codes, self.absmax, self.bf16, self.absmax_q,
                            self.absmax_scale, bias)

    @classmethod
    def nf4(cls, w_bf16, stream=None):
        codes, absmax = nf4_quantize(w_bf16, stream)
        return cls(w_bf16.shape[0], w_bf16.shape[1], codes=codes, absmax=absmax)

    @classmethod
    def nf4dq(cls, w_bf16, stream=None):
        codes, absmax = nf4_quantize(w_bf16, stream)
        q, scale = nf4dq_quantize_absmax(absmax, stream)
        return cls(w_bf16.shape[0], w_bf16.shape[1], codes=codes, absmax_q=q, absmax_scale=scale)

    @classmethod
    def dense(cls, w_bf16):
        return cls(w_bf16.shape[0], w_bf16.shape[1], bf16=w_bf16)


# ------------------------------------------------------------------ LoRA linear
def lora_linear_workspace_bytes(T, n_out, k_in, r):
    return lib().lsl_lora_linear_workspace_bytes(T, n_out, k_in, r)


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def lora_linear_fwd(x, W, A, B, scale, ws=None, stream=None):
    T = x.shape[0]
    r = A.shape[0]
    y = torch.empty((T, W.n_out), dtype=torch.bfloat16, device=x.device)
    t = torch.empty((T, r), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _ws(lora_linear_workspace_bytes(T, W.n_out, W.k_in, r), x.device)
    _check("lora_linear_fwd", lib().lora_linear_fwd(_p(x), T, C.byref(W.struct), _p(A), _p(B), r, scale,
                                                    _p(y), _p(t), _p(ws), ws.numel(), _s(stream)))
    return y, t


def lora_linear_fwd_noalloc(x, W, A, B, scale, y=None, t=None, stream=None):
    """lora_linear_fwd with the library's own device scratch (no workspace)."""
    T = x.shape[0]
    r = A.shape[0]
    if y is None:
        y = torch.empty((T, W.n_out), dtype=torch.bfloat16, device=x.device)
    if t is None:
        t = torch.empty((T, r), dtype=torch.bfloat16, device=x.device)
    _check("lora_linear_fwd_noalloc", lib().lora_linear_fwd_noalloc(_p(x), T, C.byref(W.struct), _p(A), _p(B), r,
                                                                    scale, _p(y), _p(t), _s(stream)))
    return y, t


def noalloc_scratch_bytes():
    return lib().lsl_noalloc_scratch_bytes()


def lora_linear_bwd_u(ws, T, W, r):
    """The u = bf16(dy B) [T x r] that lora_linear_bwd left in its workspace ws."""
    off = lib().lsl_lora_linear_bwd_u_offset(T, W.n_out, W.k_in)
    return ws[off:off + T * r * 2].view(torch.bfloat16).view(T, r)


def lora_linear_bwd(x, t, dy, W, A, B, scale, dA, dB, need_dx=True, ws=None, stream=None):
    T = x.shape[0]
    r = A.shape[0]
    dx = torch.empty((T, W.k_in), dtype=torch.bfloat16, device=x.device) if need_dx else None
    if ws is None:
        ws = _ws(lora_linear_workspace_bytes(T, W.n_out, W.k_in, r), x.device)
    _check("lora_linear_bwd", lib().lora_linear_bwd(_p(x), _p(t), _p(dy), T, C.byref(W.struct), _p(A), _p(B), r,
                                                    scale, _p(dx), _p(dA), _p(dB), _p(ws), ws.numel(), _s(stream)))
    return dx


# ------------------------------------------------------------------ support ops
def rmsnorm_fwd(x, w, eps, stream=None):
    T, H = x.shape
    y = torch.empty_like(x)
    _check("lsl_rmsnorm_fwd", lib().lsl_rmsnorm_fwd(_p(x), _p(w), T, H, eps, _p(y), _s(stream)))
    return y


def rmsnorm_bwd(x, w, dy, eps, dres=None, stream=None):
    T, H = x.shape
    dx = torch.empty_like(x)
    _check("lsl_rmsnorm_bwd", lib().lsl_rmsnorm_bwd(_p(x), _p(w), _p(dy), _p(dres), T, H, eps, _p(dx), _s(stream)))
    return dx


def rope_scaling(scaling):
    """(factor, low_freq_factor, high_freq_factor, original_max_position) or None
    -> ctypes lsl_rope_scaling (factor 0 = none)."""
    return _abi.RopeScaling(*(scaling if scaling else (0.0, 0.0, 0.0, 0.0)))


def rope(x, n_heads, head_dim, seq, theta, inverse=False, stream=None, scaling=None):
    """In place on x [T x ld] (bf16)."""
    T, ld = x.shape
    sc = rope_scaling(scaling)
    _check("lsl_rope", lib().lsl_rope(_p(x), T, ld, n_heads, head_dim, seq, theta, C.byref(sc), int(inverse),
                                      _s(stream)))
    return x


def swiglu_fwd(gu, stream=None):
    T, I2 = gu.shape
    a = torch.empty((T, I2 // 2), dtype=gu.dtype, device=gu.device)
    _check("lsl_swiglu_fwd", lib().lsl_swiglu_fwd(_p(gu), T, I2 // 2, _p(a), _s(stream)))
    return a


def swiglu_bwd(gu, da, stream=None):
    T, I2 = gu.shape
    dgu = torch.empty_like(gu)
    _check("lsl_swiglu_bwd", lib().lsl_swiglu_bwd(_p(gu), _p(da), T, I2 // 2, _p(dgu), _s(stream)))
    return dgu


def embed_fwd(table, ids, stream=None):
    V, H = table.shape
    T = ids.shape[0]
    out = torch.empty((T, H), dtype=table.dtype, device=table.device)
    _check("lsl_embed_fwd", lib().lsl_embed_fwd(_p(table), _p(ids), T, H, V, _p(out), _s(stream)))
    return out


def adamw_step(p, p_bf16, g, m, v, step, lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, stream=None):
    _check("lsl_adamw_step", lib().lsl_adamw_step(_p(p), _p(p_bf16), _p(g), _p(m), _p(v), p.numel(), step, lr,
                                                  beta1, beta2, eps, weight_decay, _s(stream)))


def attention_fwd(q, k, v, batch, seq, n_q, n_kv, head_dim, want_o32=False, stream=None):
    """q [T x ldq], k, v [T x ldk] views with unit column stride -> (o [T x n_q d], lse [batch x n_q x seq], o32)."""
    T = batch * seq
    o = torch.empty((T, n_q * head_dim), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((batch, n_q, seq), dtype=torch.float32, device=q.device)
    o32 = torch.empty((T, n_q * head_dim), dtype=torch.float32, device=q.device) if want_o32 else None
    _check("lsl_attention_fwd", lib().lsl_attention_fwd(_p(q), _p(k), _p(v), q.stride(0), k.stride(0), batch, seq,
                                                        n_q, n_kv, head_dim, _p(o), o.stride(0), _p(lse), _p(o32),
                                                        _s(stream)))
    return o, lse, o32


def attention_bwd(q, k, v, o, do, lse, batch, seq, n_q, n_kv, head_dim, o32=None, stream=None):
    T = batch * seq
    dq = torch.empty((T, n_q * head_dim), dtype=torch.bfloat16, device=q.device)
    dk = torch.empty((T, n_kv * head_dim), dtype=torch.bfloat16, device=q.device)
    dv = torch.empty((T, n_kv * head_dim), dtype=torch.bfloat16, device=q.device)
    ws = _ws(lib().lsl_attention_workspace_bytes(batch, seq, n_q, n_kv, head_dim), q.device)
    if q.stride(0) != dq.stride(0) or k.stride(0) != dk.stride(0) or o.stride(0) != do.stride(0):
        raise ValueError("attention_bwd: q/k must be densely packed for this wrapper")
    _check("lsl_attention_bwd", lib().lsl_attention_bwd(_p(q), _p(k), _p(v), _p(o), _p(do), _p(lse), _p(o32),
                                                        q.stride(0),
                                                        k.stride(0), o.stride(0), batch, seq, n_q, n_kv, head_dim,
                                                        _p(dq), _p(dk),
                                                        _p(dv), _p(ws), ws.numel(), _s(stream)))
    return dq, dk, dv


# ------------------------------------------------------------------ cross-entropy
def ce_workspace_bytes(T, H, V):
    return lib().lsl_ce_workspace_bytes(T, H, V)


def fused_ce_loss_fwd(hN, w_lm, labels, ignore_index=-100, ws=None, stream=None):
    """-> (loss float32 [1] on device, lse float32 [T])."""
    T, H = hN.shape
    V = w_lm.shape[0]
    loss = torch.empty(1, dtype=torch.float32, device=hN.device)
    lse = torch.empty(T, dtype=torch.float32, device=hN.device)
    if ws is None:
        ws = _ws(ce_workspace_bytes(T, H, V), hN.device)
    _check("fused_ce_loss_fwd", lib().fused_ce_loss_fwd(_p(hN), _p(w_lm), _p(labels), T, H, V, ignore_index, _p(loss),
                                                        _p(lse), _p(ws), ws.numel(), _s(stream)))
    return loss, lse


def fused_ce_logprobs(hN, w_lm, labels, batch, ignore_index=-100, ws=None, logp=None, seq_logp=None, stream=None):
    """-> (logp float32 [T], seq_logp float32 [batch]) on the device."""
    T, H = hN.shape
    V = w_lm.shape[0]
    if logp is None:
        logp = torch.empty(T, dtype=torch.float32, device=hN.device)
    if seq_logp is None:
        seq_logp = torch.empty(batch, dtype=torch.float32, device=hN.device)
    if ws is None:
        ws = _ws(ce_workspace_bytes(T, H, V), hN.device)
    _check("fused_ce_logprobs", lib().fused_ce_logprobs(_p(hN), _p(w_lm), _p(labels), T, H, V, ignore_index, batch,
                                                        _p(logp), _p(seq_logp), _p(ws), ws.numel(), _s(stream)))
    return logp, seq_logp


def fused_ce_loss_bwd(hN, w_lm, labels, lse, grad_scale=1.0, ignore_index=-100, ws=None, out=None, stream=None):
    T, H = hN.shape
    V = w_lm.shape[0]
    dh = torch.empty_like(hN) if out is None else out
    if ws is None:
        ws = _ws(ce_workspace_bytes(T, H, V), hN.device)
    _check("fused_ce_loss_bwd", lib().fused_ce_loss_bwd(_p(hN), _p(w_lm), _p(labels), _p(lse), T, H, V, ignore_index,
                                                        grad_scale, _p(dh), _p(ws), ws.numel(), _s(stream)))
    return dh
