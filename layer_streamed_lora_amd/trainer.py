"""One LoRA training step of a decoder-only model whose frozen layers are
streamed from a pinned host store through a two-slot HBM pool, or kept
resident in HBM (the reference the streamed run must equal bit for bit).

The method ("Exact Layer Streaming ...", abstract; "Soup CLI ...", section
"How Layer Streaming Works"): the base stays in host RAM and one decoder layer
at a time is brought to the GPU for the forward and again for the backward;
only layer-boundary activations are kept and each layer is recomputed in its
backward. Gradient accumulation re-streams every layer per microbatch, which
costs the same bytes per token whatever the microbatch count.

Scheduling: the layer visit order is 0..L-1 (forward), L-1..0 (backward), then
the next microbatch. Visit i computes on one slot while the layer of visit
i + 1 is copied into the other (copy stream, ordered by the pool's events).
Layers already in a slot at the turn of a sweep (forward to backward, and
backward to the next microbatch's forward) are reused without a copy, so a
microbatch costs 2L - 4 copies (2L - 2 for the very first one). The selection of kernels
never depends on where a layer lives, so both modes run identical arithmetic.
"""
import ctypes as C

import numpy as np
import torch

from . import _abi
from .model import LoraParams, layer_cfg, layer_layout, write_layer_blob, layer_workspace_bytes, layer_tkeep_bytes
from .ops import lib, _check, _p, _s, embed_fwd, rmsnorm_fwd, rmsnorm_bwd, fused_ce_loss_fwd, fused_ce_loss_bwd
from .ops import ce_workspace_bytes, adamw_step

IGNORE = -100


def shifted_labels(ids, batch, seq):
    lab = np.full((batch, seq), IGNORE, np.int32)
    lab[:, :-1] = np.asarray(ids).reshape(batch, seq)[:, 1:]
    return lab.reshape(-1)


_COPY_STREAMS = {}


def copy_stream(device="cuda"):
    """The one stream every layer pool of this process copies on (per device).

    HIP maps streams onto a few hardware queues (GPU_MAX_HW_QUEUES, 4 by
    default); two streams that share a queue run one after the other, so a copy
    stream that lands on the compute stream's queue stops overlapping with it
    (a streamed step then costs copies plus compute). This stream is created
    directly as a non-blocking HIP stream, so torch's pool of 32+ streams is not
    initialised by this package and the process keeps two streams: the compute
    stream and this one. It lives until the process ends."""
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    if idx not in _COPY_STREAMS:
        hip = C.CDLL("libamdhip64.so")
        handle = C.c_void_p()
        with torch.cuda.device(idx):
            rc = hip.hipStreamCreateWithFlags(C.byref(handle), C.c_uint(1))  # hipStreamNonBlocking
        if rc != 0:
            raise RuntimeError(f"hipStreamCreateWithFlags failed with HIP error {rc}")
        _COPY_STREAMS[idx] = torch.cuda.ExternalStream(handle.value, device=idx)
    return _COPY_STREAMS[idx]


class LayerPool:
    """Python handle of the C pool (slots are device tensors owned here)."""

    def __init__(self, n_slots, slot_bytes, device="cuda"):
        self.slot_bytes = slot_bytes
        self.copy_stream = copy_stream(device)
        self.slots = [torch.empty(slot_bytes, dtype=torch.uint8, device=device) for _ in range(n_slots)]
        ptrs = (C.c_void_p * n_slots)(*[s.data_ptr() for s in self.slots])
        self.handle = C.c_void_p()
        _check("lsl_pool_create", lib().lsl_pool_create(C.byref(self.handle), ptrs, n_slots, slot_bytes,
                                                        self.copy_stream.cuda_stream))

    def load(self, slot, host_view):
        _check("load_layer_async", lib().load_layer_async(self.handle, slot, host_view.data_ptr(), host_view.numel()))

    def acquire(self, slot, stream=None):
        p = C.c_void_p()
        _check("lsl_pool_acquire", lib().lsl_pool_acquire(self.handle, slot, _s(stream), C.byref(p)))
        return p.value

    def release(self, slot, stream=None):
        _check("lsl_pool_release", lib().lsl_pool_release(self.handle, slot, _s(stream)))

    def reuse(self, slot):
        _check("lsl_pool_reuse", lib().lsl_pool_reuse(self.handle, slot))

    def close(self):
        if self.handle:
            lib().lsl_pool_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StreamedLoraModel:
    """Frozen decoder-only base (layer blobs, embedding, final norm, lm_head) with
    trainable LoRA adapters on every projection of every layer.

    mode: "streamed" (pinned host store + 2-slot pool) or "resident" (all
    blobs in HBM). Both share the same blob bytes, adapters and kernels."""

    def __init__(self, shape, n_layers, vocab, tied, batch, seq, mode="streamed", device="cuda", keep_t=True):
        """keep_t: each layer's forward keeps its LoRA products t (rank-r per
        token and projection) for the backward's recompute, which then skips
        computing them again (the same bits either way)."""
        assert mode in ("streamed", "resident")
        self.shape, self.n_layers, self.vocab, self.tied = shape, n_layers, vocab, tied
        self.batch, self.seq, self.T = batch, seq, batch * seq
        self.mode, self.device = mode, device
        self.cfg = layer_cfg(shape)
        self.layout = layer_layout(self.cfg)
        self.blob_bytes = int(self.layout.total_bytes)
        self.stride = (self.blob_bytes + 4095) // 4096 * 4096
        H = shape.hidden
        if mode == "streamed":
            self.store = torch.empty(n_layers * self.stride, dtype=torch.uint8, pin_memory=True)
            self.pool = LayerPool(2, self.blob_bytes, device)
        else:
            self.store = torch.empty(n_layers * self.stride, dtype=torch.uint8, device=device)
            self.pool = None
        self.embed = torch.empty((vocab, H), dtype=torch.bfloat16, device=device)
        self.final_norm = torch.ones(H, dtype=torch.bfloat16, device=device)
        self.lm_head = None if tied else torch.empty((vocab, H), dtype=torch.bfloat16, device=device)
        self.lora = LoraParams(shape, n_layers, device)
        T = self.T
        self.ckpt = torch.empty((n_layers + 1, T, H), dtype=torch.bfloat16, device=device)
        self.hn = torch.empty((T, H), dtype=torch.bfloat16, device=device)
        self.dh = [torch.empty((T, H), dtype=torch.bfloat16, device=device) for _ in range(2)]
        self.ws = torch.empty(max(layer_workspace_bytes(self.cfg, batch, seq, _abi.MODE_BWD),
                                  ce_workspace_bytes(T, H, vocab), 256), dtype=torch.uint8, device=device)
        self.lse = torch.empty(T, dtype=torch.float32, device=device)
        tk = layer_tkeep_bytes(self.cfg, batch, seq)  # a multiple of 256: every row stays aligned
        self.tkeep = torch.empty((n_layers, tk), dtype=torch.uint8, device=device) if keep_t else None
        self.step_count = 0
        self.slot_layer = [None, None]
        self._released = [False, False]
        self.h2d_bytes = 0
        self.loads = 0

    # ------------------------------------------------------------ building
    def blob_view(self, layer):
        return self.store[layer * self.stride: layer * self.stride + self.blob_bytes]

    def set_layer_weights(self, layer, w):
        """w: dict of cuda bf16 tensors ('q'.. 'down' [out x in], 'norm1', 'norm2', and
        'q_bias', 'k_bias', 'v_bias' when the shape has them)."""
        if self.mode == "resident":
            write_layer_blob(self.shape, self.cfg, self.blob_view(layer), w)
        else:
            tmp = torch.empty(self.blob_bytes, dtype=torch.uint8, device=self.device)
            write_layer_blob(self.shape, self.cfg, tmp, w)
            self.blob_view(layer).copy_(tmp)
        torch.cuda.synchronize()

    def copy_base_from(self, other):
        """Share the frozen base bytes and the adapters of another model."""
        self.store.copy_(other.store)
        self.embed.copy_(other.embed)
        self.final_norm.copy_(other.final_norm)
        if self.lm_head is not None:
            self.lm_head.copy_(other.lm_head)
        for name in ("master", "bf16", "grad", "m", "v"):
            getattr(self.lora, name).copy_(getattr(other.lora, name))
        self.step_count = other.step_count
        torch.cuda.synchronize()

    @property
    def w_lm(self):
        return self.embed if self.tied else self.lm_head

    # ------------------------------------------------------------ streaming
    def _blob_ptr_for_visit(self, seq_layers, i):
        """Make layer seq_layers[i] available; prefetch the next visit's layer."""
        l = seq_layers[i]
        if self.mode == "resident":
            return self.blob_view(l).data_ptr(), None
        s = self.slot_layer.index(l) if l in self.slot_layer else None
        if s is None:  # only the very first visit of a run lands here
            s = 0
            self._load(s, l)
        if i + 1 < len(seq_layers):
            ln = seq_layers[i + 1]
            if ln not in self.slot_layer:
                self._load(1 - s, ln)
        if self._released[s]:
            self.pool.reuse(s)
        ptr = self.pool.acquire(s)
        return ptr, s

    def _load(self, slot, layer):
        self.pool.load(slot, self.blob_view(layer))
        self.slot_layer[slot] = layer
        self._released[slot] = False
        self.h2d_bytes += self.blob_bytes
        self.loads += 1

    def _tkeep(self, layer):
        return None if self.tkeep is None else self.tkeep[layer].data_ptr()

    def _done(self, slot):
        if slot is not None:
            self.pool.release(slot)
            self._released[slot] = True

    # ------------------------------------------------------------ step
    def prepare_inputs(self, id_chunks):
        """Token ids (list of [batch*seq] arrays, one per microbatch) -> device
        tensors (ids, shifted labels), each [n_micro x T] int32."""
        ids = np.stack([np.asarray(c, np.int32).reshape(-1) for c in id_chunks])
        labels = np.stack([shifted_labels(c, self.batch, self.seq) for c in id_chunks])
        return (torch.from_numpy(ids).to(self.device), torch.from_numpy(labels).to(self.device))

    def microbatch(self, ids, labels, loss_out, grad_scale):
        """Forward + backward of one microbatch (device ids/labels [T]); adds
        grad_scale * gradient into the adapter gradients, writes the microbatch
        loss into loss_out (one float on the device)."""
        L, T, H = self.n_layers, self.T, self.shape.hidden
        stream = torch.cuda.current_stream()
        _check("lsl_embed_fwd", lib().lsl_embed_fwd(_p(self.embed), _p(ids), T, H, self.vocab,
                                                    _p(self.ckpt[0]), _s(stream)))
        visits = list(range(L)) + list(range(L - 1, -1, -1))
        cfg = self.cfg
        for i in range(L):
            ptr, slot = self._blob_ptr_for_visit(visits, i)
            _check("decoder_layer_fwd", lib().decoder_layer_fwd(
                C.byref(cfg), ptr, C.byref(self.lora.lora_set(i)), _p(self.ckpt[i]), self.batch, self.seq,
                _p(self.ckpt[i + 1]), self._tkeep(i), _p(self.ws), self.ws.numel(), _s(stream)))
            self._done(slot)
        eps = self.shape.rms_eps
        _check("lsl_rmsnorm_fwd", lib().lsl_rmsnorm_fwd(_p(self.ckpt[L]), _p(self.final_norm), T, H, eps,
                                                        _p(self.hn), _s(stream)))
        _check("fused_ce_loss_fwd", lib().fused_ce_loss_fwd(_p(self.hn), _p(self.w_lm), _p(labels), T, H,
                                                            self.vocab, IGNORE, _p(loss_out), _p(self.lse),
                                                            _p(self.ws), self.ws.numel(), _s(stream)))
        dhn = self.dh[1]
        _check("fused_ce_loss_bwd", lib().fused_ce_loss_bwd(_p(self.hn), _p(self.w_lm), _p(labels),
                                                            _p(self.lse), T, H, self.vocab, IGNORE, grad_scale,
                                                            _p(dhn), _p(self.ws), self.ws.numel(), _s(stream)))
        dh = self.dh[0]
        _check("lsl_rmsnorm_bwd", lib().lsl_rmsnorm_bwd(_p(self.ckpt[L]), _p(self.final_norm), _p(dhn), None, T, H,
                                                        eps, _p(dh), _s(stream)))
        cur = 0
        for j in range(L):
            i = L + j
            layer = visits[i]
            ptr, slot = self._blob_ptr_for_visit(visits, i)
            dx = self.dh[1 - cur] if layer > 0 else None
            _check("decoder_layer_bwd", lib().decoder_layer_bwd(
                C.byref(cfg), ptr, C.byref(self.lora.lora_set(layer)), _p(self.ckpt[layer]), _p(self.dh[cur]),
                self.batch, self.seq, _p(dx), C.byref(self.lora.lora_grads(layer)), self._tkeep(layer), _p(self.ws),
                self.ws.numel(), _s(stream)))
            self._done(slot)
            cur = 1 - cur

    def reference_logprobs(self, inputs):
        """Forward-only sweep of every microbatch through the frozen base with the
        adapters off (layer calls with no LoRA set), then the per-token and
        per-sequence log-probabilities of the shifted labels. Returns device
        tensors (logp [n_micro x T], seq_logp [n_micro x batch]); each microbatch
        streams every layer once, in order."""
        ids, labels = inputs
        n = ids.shape[0]
        L, T, H = self.n_layers, self.T, self.shape.hidden
        stream = torch.cuda.current_stream()
        logp = torch.empty((n, T), dtype=torch.float32, device=self.device)
        seq_logp = torch.empty((n, self.batch), dtype=torch.float32, device=self.device)
        visits = list(range(L))
        cfg = self.cfg
        for mb in range(n):
            _check("lsl_embed_fwd", lib().lsl_embed_fwd(_p(self.embed), _p(ids[mb]), T, H, self.vocab,
                                                        _p(self.ckpt[0]), _s(stream)))
            for i in range(L):
                ptr, slot = self._blob_ptr_for_visit(visits, i)
                # ping-pong between two checkpoint rows: only the last hidden state is needed
                src, dst = self.ckpt[i % 2], self.ckpt[(i + 1) % 2]
                _check("decoder_layer_fwd", lib().decoder_layer_fwd(
                    C.byref(cfg), ptr, None, _p(src), self.batch, self.seq, _p(dst), None, _p(self.ws),
                    self.ws.numel(), _s(stream)))
                self._done(slot)
            _check("lsl_rmsnorm_fwd", lib().lsl_rmsnorm_fwd(_p(self.ckpt[L % 2]), _p(self.final_norm), T, H,
                                                            self.shape.rms_eps, _p(self.hn), _s(stream)))
            _check("fused_ce_logprobs", lib().fused_ce_logprobs(
                _p(self.hn), _p(self.w_lm), _p(labels[mb]), T, H, self.vocab, IGNORE, self.batch, _p(logp[mb]),
                _p(seq_logp[mb]), _p(self.ws), self.ws.numel(), _s(stream)))
        return logp, seq_logp

    def step(self, inputs, lr=2e-4, adamw=True):
        """One optimizer step over the microbatches of `inputs` (from
        prepare_inputs). Returns the per-microbatch losses as a device tensor
        (no host synchronisation); the step's loss is their mean."""
        ids, labels = inputs
        n = ids.shape[0]
        losses = torch.empty(n, dtype=torch.float32, device=self.device)
        self.lora.grad.zero_()
        for i in range(n):
            self.microbatch(ids[i], labels[i], losses[i:i + 1], 1.0 / n)
        if adamw:
            self.step_count += 1
            adamw_step(self.lora.master, self.lora.bf16, self.lora.grad, self.lora.m, self.lora.v, self.step_count,
                       lr=lr)
        return losses
