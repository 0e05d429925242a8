"""Host-side structures of the streamed model: layer configs, packed layer
blobs (the unit the pool streams), LoRA parameter sets and their gradients and
optimizer state. Memory comes from torch; all arithmetic runs in liblsl.so."""
import ctypes as C

import torch

from . import _abi
from .ops import lib, _check, _p, _s

PROJ_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
WFMT_CODES = {"nf4": _abi.WFMT_NF4, "bf16": _abi.WFMT_BF16, "nf4dq": _abi.WFMT_NF4DQ}


def layer_cfg(shape):
    """ctypes lsl_layer_cfg from a synth LayerShape-like object."""
    from .ops import rope_scaling
    return _abi.LayerCfg(shape.hidden, shape.n_q, shape.n_kv, shape.head_dim, shape.inter, shape.rms_eps,
                         shape.rope_theta, WFMT_CODES[shape.wfmt],
                         shape.lora_r, shape.lora_alpha / shape.lora_r,
                         int(bool(getattr(shape, "qkv_bias", False))),
                         rope_scaling(getattr(shape, "rope_scaling", None)))


def layer_layout(cfg):
    L = _abi.LayerLayout()
    _check("lsl_layer_layout_get", lib().lsl_layer_layout_get(C.byref(cfg), C.byref(L)))
    return L


def mat_shapes(shape):
    q, kv = shape.n_q * shape.head_dim, shape.n_kv * shape.head_dim
    return [(q + 2 * kv, shape.hidden), (shape.hidden, q), (2 * shape.inter, shape.hidden), (shape.hidden, shape.inter)]


def write_layer_blob(shape, cfg, blob, w, stream=None):
    """Fill a device uint8 blob [total_bytes] from bf16 weights w (dict of cuda
    bf16 tensors 'q','k','v','o','gate','up','down' [out x in], 'norm1', 'norm2').
    NF4 matrices are quantised on the GPU straight into the blob."""
    L = layer_layout(cfg)
    assert blob.numel() >= L.total_bytes and blob.dtype == torch.uint8

    def region(off, nbytes):
        return blob[off:off + nbytes]
    region(L.norm1_off, 2 * shape.hidden).view(torch.bfloat16).copy_(w["norm1"])
    region(L.norm2_off, 2 * shape.hidden).view(torch.bfloat16).copy_(w["norm2"])
    if cfg.qkv_bias:
        b = torch.cat([w["q_bias"], w["k_bias"], w["v_bias"]]).contiguous()
        region(L.bias_off, 2 * b.numel()).view(torch.bfloat16).copy_(b)
    for i, (names, (n, k)) in enumerate(zip(PROJ_GROUPS, mat_shapes(shape))):
        m = torch.cat([w[nm] for nm in names], dim=0).contiguous()
        assert m.shape == (n, k)
        if cfg.wfmt == _abi.WFMT_NF4:
            codes = region(L.w_off[i], n * k // 2)
            absmax = region(L.absmax_off[i], n * k // 64 * 4).view(torch.float32)
            _check("lsl_nf4_quantize", lib().lsl_nf4_quantize(_p(m), n, k, _p(codes), _p(absmax), _s(stream)))
        elif cfg.wfmt == _abi.WFMT_NF4DQ:
            nb = n * k // 64
            codes = region(L.w_off[i], n * k // 2)
            absmax = torch.empty(nb, dtype=torch.float32, device=blob.device)
            _check("lsl_nf4_quantize", lib().lsl_nf4_quantize(_p(m), n, k, _p(codes), _p(absmax), _s(stream)))
            q = region(L.absmax_off[i], nb)
            scale = region(L.scale_off[i], (nb + 255) // 256 * 4).view(torch.float32)
            _check("lsl_nf4dq_quantize_absmax",
                   lib().lsl_nf4dq_quantize_absmax(_p(absmax), nb, _p(q), _p(scale), _s(stream)))
        else:
            region(L.w_off[i], n * k * 2).view(torch.bfloat16).copy_(m.view(-1))
    return L


def _pad8(n):
    return (n + 7) // 8 * 8


class LoraParams:
    """All adapters of a model in flat buffers: fp32 master, bf16 working copy,
    fp32 gradient and AdamW moments. Per layer, per fused group i, A[i] and B[i]
    are views (16-byte aligned) into the flat buffers."""

    def __init__(self, shape, n_layers, device="cuda"):
        r = shape.lora_r
        q, kv, H, I = shape.n_q * shape.head_dim, shape.n_kv * shape.head_dim, shape.hidden, shape.inter
        self.shapes = [((3 * r, H), (q + 2 * kv, r)), ((r, q), (H, r)), ((2 * r, H), (2 * I, r)), ((r, I), (H, r))]
        self.out_rows = {"q": q, "k": kv, "v": kv, "o": H, "gate": I, "up": I, "down": H}
        per_layer = sum(_pad8(a[0] * a[1]) + _pad8(b[0] * b[1]) for a, b in self.shapes)
        self.n_layers = n_layers
        self.numel = per_layer * n_layers
        self.master = torch.zeros(self.numel, dtype=torch.float32, device=device)
        self.bf16 = torch.zeros(self.numel, dtype=torch.bfloat16, device=device)
        self.grad = torch.zeros(self.numel, dtype=torch.float32, device=device)
        self.m = torch.zeros(self.numel, dtype=torch.float32, device=device)
        self.v = torch.zeros(self.numel, dtype=torch.float32, device=device)
        self.offsets = []  # per layer: [(offA, offB)] * 4
        off = 0
        for _ in range(n_layers):
            lay = []
            for a, b in self.shapes:
                oa = off
                off += _pad8(a[0] * a[1])
                ob = off
                off += _pad8(b[0] * b[1])
                lay.append((oa, ob))
            self.offsets.append(lay)
        self._sets = [None] * n_layers
        self._grads = [None] * n_layers

    def view(self, buf, layer, i, which):
        oa, ob = self.offsets[layer][i]
        a, b = self.shapes[i]
        if which == "A":
            return buf[oa:oa + a[0] * a[1]].view(a)
        return buf[ob:ob + b[0] * b[1]].view(b)

    def set_from(self, layer, lora_np, names_by_group=PROJ_GROUPS):
        """Load per-projection arrays 'A_p', 'B_p' (numpy, bf16-exact float32)."""
        import numpy as np
        for i, names in enumerate(names_by_group):
            A = np.concatenate([lora_np["A_" + n] for n in names], axis=0)
            B = np.concatenate([lora_np["B_" + n] for n in names], axis=0)
            self.view(self.master, layer, i, "A").copy_(torch.from_numpy(A))
            self.view(self.master, layer, i, "B").copy_(torch.from_numpy(B))
        self.bf16.copy_(self.master.to(torch.bfloat16))

    def lora_set(self, layer):
        if self._sets[layer] is None:
            s = _abi.LoraSet()
            for i in range(4):
                s.A[i] = _p(self.view(self.bf16, layer, i, "A"))
                s.B[i] = _p(self.view(self.bf16, layer, i, "B"))
            self._sets[layer] = s
        return self._sets[layer]

    def lora_grads(self, layer):
        if self._grads[layer] is None:
            g = _abi.LoraGrads()
            for i in range(4):
                g.dA[i] = _p(self.view(self.grad, layer, i, "A"))
                g.dB[i] = _p(self.view(self.grad, layer, i, "B"))
            self._grads[layer] = g
        return self._grads[layer]

    def grads_np(self, layer, names_by_group=PROJ_GROUPS):
        """Per-projection gradients of one layer as float64 numpy arrays."""
        out = {}
        for i, names in enumerate(names_by_group):
            dA = self.view(self.grad, layer, i, "A").double().cpu().numpy()
            dB = self.view(self.grad, layer, i, "B").double().cpu().numpy()
            ra = dA.shape[0] // len(names)
            rb = 0
            for j, n in enumerate(names):
                out["A_" + n] = dA[j * ra:(j + 1) * ra]
                out["B_" + n] = dB[rb:rb + self.out_rows[n]]
                rb += self.out_rows[n]
        return out


def layer_workspace_bytes(cfg, batch, seq, mode):
    return lib().lsl_layer_workspace_bytes(C.byref(cfg), batch, seq, mode)


def layer_workspace_map(cfg, batch, seq, mode):
    """Byte offsets of the layer's intermediates inside its workspace (dict)."""
    m = _abi.LayerWsMap()
    _check("lsl_layer_workspace_map", lib().lsl_layer_workspace_map(C.byref(cfg), batch, seq, mode, C.byref(m)))
    return {n: int(getattr(m, n)) for n in _abi.WS_MAP_FIELDS}


def layer_tkeep_bytes(cfg, batch, seq):
    """Bytes of a buffer that keeps the layer forward's LoRA products t for its backward."""
    return int(lib().lsl_layer_tkeep_bytes(C.byref(cfg), batch, seq))


def decoder_layer_fwd(cfg, blob, lora_set, x, batch, seq, out=None, ws=None, t_keep=None, stream=None):
    """lora_set None: adapters off (the frozen base alone). t_keep: optional
    uint8 device buffer of layer_tkeep_bytes that receives the products t."""
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = torch.empty(layer_workspace_bytes(cfg, batch, seq, _abi.MODE_FWD), dtype=torch.uint8, device=x.device)
    lo = None if lora_set is None else C.byref(lora_set)
    _check("decoder_layer_fwd", lib().decoder_layer_fwd(C.byref(cfg), _p(blob), lo, _p(x), batch, seq,
                                                        _p(out), _p(t_keep), _p(ws), ws.numel(), _s(stream)))
    return out


def decoder_layer_bwd(cfg, blob, lora_set, x, dy, batch, seq, grads, dx=True, ws=None, t_keep=None, stream=None):
    """t_keep: the buffer decoder_layer_fwd of the same x filled (the recompute
    then takes t from it), or None (t recomputed)."""
    dxt = torch.empty_like(x) if dx is True else dx
    if ws is None:
        ws = torch.empty(layer_workspace_bytes(cfg, batch, seq, _abi.MODE_BWD), dtype=torch.uint8, device=x.device)
    _check("decoder_layer_bwd", lib().decoder_layer_bwd(C.byref(cfg), _p(blob), C.byref(lora_set), _p(x), _p(dy),
                                                        batch, seq, _p(dxt), C.byref(grads), _p(t_keep), _p(ws),
                                                        ws.numel(), _s(stream)))
    return dxt
