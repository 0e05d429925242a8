"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/lsl.h declares, and rejects bad arguments with the
documented status before touching a device."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "lsl.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


@pytest.fixture(scope="module")
def L():
    import layer_streamed_lora_amd as lsl
    return lsl


def test_header_lists_entry_points():
    names = header_functions()
    for n in ("load_layer_async", "lora_linear_fwd", "lora_linear_bwd", "decoder_layer_fwd", "decoder_layer_bwd",
              "fused_ce_loss_fwd", "fused_ce_loss_bwd", "lsl_pool_create", "lsl_nf4_quantize"):
        assert n in names
    assert len(names) >= 30


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    missing = [n for n in header_functions() if not hasattr(lib, n)]
    assert not missing, missing
    from layer_streamed_lora_amd import _abi
    assert set(_abi.PROTOS) == set(header_functions())


def test_codebook_matches_oracle_bitwise(L):
    from oracle.nf4 import nf4_codebook
    got = np.array(L.nf4_codebook(), np.float32)
    assert np.array_equal(got.view(np.uint32), nf4_codebook().view(np.uint32))


def test_abi_version(L):
    assert L.abi_version() == 3


def _status(L, name, *args):
    return getattr(L.lib(), name)(*args)


def test_validation_rejects_before_enqueue(L):
    from layer_streamed_lora_amd import _abi
    lib = L.lib()
    # non-multiple-of-64 columns
    assert lib.lsl_nf4_quantize(None, 4, 63, None, None, None) == _abi.LSL_ERR_INVALID_ARG
    assert b"multiple of 64" in lib.lsl_last_error()
    # null weight
    assert lib.lora_linear_fwd(None, 8, None, None, None, 8, 2.0, None, None, None, 0, None) == _abi.LSL_ERR_INVALID_ARG
    # rank not a multiple of 8
    w = _abi.Weight(_abi.WFMT_BF16, 0, 64, 64, None, None, 16)
    assert lib.lora_linear_fwd(16, 8, C.byref(w), 16, 16, 12, 2.0, 16, 16, None, 0, None) == _abi.LSL_ERR_UNSUPPORTED
    # k_in not a multiple of 64
    w = _abi.Weight(_abi.WFMT_BF16, 0, 64, 96, None, None, 16)
    assert lib.lora_linear_fwd(16, 8, C.byref(w), 16, 16, 8, 2.0, 16, 16, None, 0, None) == _abi.LSL_ERR_UNSUPPORTED
    w = _abi.Weight(_abi.WFMT_BF16, 0, 72, 64, None, None, 16)
    assert lib.lora_linear_fwd(16, 8, C.byref(w), 16, 16, 8, 2.0, 16, 16, None, 0, None) == _abi.LSL_ERR_UNSUPPORTED
    # NF4 weight with a bf16 pointer set
    w = _abi.Weight(_abi.WFMT_NF4, 0, 64, 64, 256, 256, 256)
    assert lib.lora_linear_fwd(16, 8, C.byref(w), 16, 16, 8, 2.0, 16, 16, None, 0, None) == _abi.LSL_ERR_INVALID_ARG
    # misaligned activation pointer
    w = _abi.Weight(_abi.WFMT_BF16, 0, 64, 64, None, None, 256)
    assert lib.lora_linear_fwd(18, 8, C.byref(w), 256, 256, 8, 2.0, 256, 256, None, 0, None) == _abi.LSL_ERR_INVALID_ARG
    # workspace too small
    assert lib.lora_linear_fwd(256, 8, C.byref(w), 256, 256, 8, 2.0, 256, 256, 256, 0, None) == _abi.LSL_ERR_WORKSPACE
    # empty input is a no-op
    assert lib.lora_linear_fwd(None, 0, C.byref(w), None, None, 8, 2.0, None, None, None, 0, None) == _abi.LSL_OK
    # pool arguments
    out = C.c_void_p()
    assert lib.lsl_pool_create(C.byref(out), None, 2, 1024, None) == _abi.LSL_ERR_INVALID_ARG
    slots = (C.c_void_p * 2)(256, 300)
    assert lib.lsl_pool_create(C.byref(out), slots, 2, 1024, None) == _abi.LSL_ERR_INVALID_ARG
    assert lib.load_layer_async(None, 0, 4096, 16) == _abi.LSL_ERR_INVALID_ARG
    assert lib.lsl_adamw_step(None, None, None, None, None, 10, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == _abi.LSL_ERR_INVALID_ARG


def test_workspace_sizes_are_deterministic(L):
    a = L.lora_linear_workspace_bytes(512, 4096, 4096, 16)
    b = L.lora_linear_workspace_bytes(512, 4096, 4096, 16)
    assert a == b and a > 0
    assert L.lora_linear_workspace_bytes(512, 4096, 4096, 12) == 0


def test_linear_workspace_covers_stream_k_and_u(L):
    """A GEMM with fewer 256 x 256 output tiles than the 256 stream-K
    workgroups (1000 tokens of a 6144 x 4096 projection: 96 tiles) keeps one
    float32 tile of partials per slot, 256 + 96 - 1 slots; the backward's u
    [T x r] region lies inside the workspace, 256-byte aligned."""
    lib = L.lib()
    T, n_out, k_in, r = 1000, 6144, 4096, 16
    ws = L.lora_linear_workspace_bytes(T, n_out, k_in, r)
    assert ws >= (256 + 96 - 1) * 256 * 256 * 4
    off = lib.lsl_lora_linear_bwd_u_offset(T, n_out, k_in)
    assert off % 256 == 0 and 0 < off and off + T * r * 2 <= ws
    assert lib.lsl_lora_linear_bwd_u_offset(0, n_out, k_in) == 0


def test_linear_workspace_split_k(L):
    """A 64-row-tile GEMM with its reduction split (300 tokens of a 6144 x 4096
    projection: 3 x 96 tiles, 2 splits) needs the splits' float32 partials,
    not stream-K slots."""
    T, n_out, k_in = 300, 6144, 4096
    ws = L.lora_linear_workspace_bytes(T, n_out, k_in, 16)
    assert 2 * T * n_out * 4 <= ws < 2 * T * n_out * 4 + (1 << 20)


def test_nf4dq_validation(L):
    from layer_streamed_lora_amd import _abi
    lib = L.lib()
    assert lib.lsl_nf4dq_quantize_absmax(None, -1, None, None, None) == _abi.LSL_ERR_INVALID_ARG
    assert lib.lsl_nf4dq_quantize_absmax(None, 0, None, None, None) == _abi.LSL_OK
    assert lib.lsl_nf4dq_quantize_absmax(256, 10, 256, None, None) == _abi.LSL_ERR_INVALID_ARG
    assert lib.lsl_nf4dq_dequant(256, 256, 256, 4, 96, 256, None) == _abi.LSL_ERR_INVALID_ARG
    # NF4DQ weight: codes + absmax_q + absmax_scale, float32 absmax and bf16 NULL
    w = _abi.Weight(_abi.WFMT_NF4DQ, 0, 64, 64, 256, 256, None, 256, 256)
    assert lib.lora_linear_fwd(256, 8, C.byref(w), 256, 256, 8, 2.0, 256, 256, None, 0, None) == _abi.LSL_ERR_INVALID_ARG
    w = _abi.Weight(_abi.WFMT_NF4DQ, 0, 64, 64, 256, None, None, 256, None)
    assert lib.lora_linear_fwd(256, 8, C.byref(w), 256, 256, 8, 2.0, 256, 256, None, 0, None) == _abi.LSL_ERR_INVALID_ARG
    w = _abi.Weight(_abi.WFMT_NF4DQ, 0, 64, 64, 256, None, None, 256, 256)
    assert lib.lora_linear_fwd(None, 0, C.byref(w), None, None, 8, 2.0, None, None, None, 0, None) == _abi.LSL_OK


@pytest.mark.parametrize("wfmt", ["nf4", "nf4dq", "bf16"])
def test_layer_layout_regions(L, wfmt):
    """The packed layer blob: every region 256-byte aligned, disjoint, inside
    total_bytes, and sized for its format; for Llama-3.1-8B NF4DQ the blob is
    the oracle's byte count plus alignment padding only (under the pages'
    113 MB buffer)."""
    import dataclasses
    from layer_streamed_lora_amd import model as M
    from synth.configs import LLAMA8B_LAYER
    from oracle.nf4 import nf4dq_layer_bytes
    shape = dataclasses.replace(LLAMA8B_LAYER, wfmt=wfmt)
    lay = M.layer_layout(M.layer_cfg(shape))
    H, I, Q, KV = shape.hidden, shape.inter, shape.q_dim, shape.kv_dim
    mats = [(Q + 2 * KV, H), (H, Q), (2 * I, H), (H, I)]
    regions = [(lay.norm1_off, 2 * H), (lay.norm2_off, 2 * H)]
    for i, (n, k) in enumerate(mats):
        nb = n * k // 64
        if wfmt == "bf16":
            regions.append((lay.w_off[i], 2 * n * k))
            assert lay.absmax_off[i] == 0 and lay.scale_off[i] == 0
        elif wfmt == "nf4":
            regions += [(lay.w_off[i], n * k // 2), (lay.absmax_off[i], 4 * nb)]
            assert lay.scale_off[i] == 0
        else:
            regions += [(lay.w_off[i], n * k // 2), (lay.absmax_off[i], nb), (lay.scale_off[i], 4 * ((nb + 255) // 256))]
    regions.sort()
    for (o, b), (o2, _) in zip(regions, regions[1:]):
        assert o % 256 == 0 and o + b <= o2
    assert regions[-1][0] + regions[-1][1] <= lay.total_bytes
    payload = sum(b for _, b in regions)
    assert lay.total_bytes - payload < 256 * len(regions)
    if wfmt == "nf4dq":
        assert payload == nf4dq_layer_bytes(H, shape.n_q, shape.n_kv, shape.head_dim, I)
        assert lay.total_bytes < 113_000_000


def test_fidelity_options_validation_and_layout(L):
    """q/k/v bias and RoPE scaling: bad options are rejected before anything is
    enqueued; the bias region is 256-byte aligned and sized [(n_q + 2 n_kv) d]."""
    import dataclasses
    from layer_streamed_lora_amd import _abi
    from layer_streamed_lora_amd import model as M
    from synth.configs import QWEN05B_LAYER, LLAMA31_ROPE_SCALING
    lib = L.lib()
    shape = dataclasses.replace(QWEN05B_LAYER, qkv_bias=True, rope_scaling=LLAMA31_ROPE_SCALING)
    cfg = M.layer_cfg(shape)
    lay = M.layer_layout(cfg)
    plain = M.layer_layout(M.layer_cfg(QWEN05B_LAYER))
    nqkv = shape.q_dim + 2 * shape.kv_dim
    assert lay.bias_off % 256 == 0 and lay.bias_off >= plain.norm2_off + 2 * shape.hidden
    assert lay.total_bytes - plain.total_bytes == (2 * nqkv + 255) // 256 * 256 and plain.bias_off == 0
    for bad in ((0.5, 1.0, 4.0, 8192.0), (8.0, 4.0, 1.0, 8192.0), (8.0, 0.0, 4.0, 8192.0), (8.0, 1.0, 4.0, 0.0)):
        c = M.layer_cfg(dataclasses.replace(shape, rope_scaling=bad))
        out = _abi.LayerLayout()
        assert lib.lsl_layer_layout_get(C.byref(c), C.byref(out)) == _abi.LSL_ERR_INVALID_ARG
        assert b"RoPE scaling" in lib.lsl_last_error()
        sc = _abi.RopeScaling(*bad)
        assert lib.lsl_rope(256, 4, 128, 1, 128, 4, 1e4, C.byref(sc), 0, None) == _abi.LSL_ERR_INVALID_ARG
    c = M.layer_cfg(shape)
    c.qkv_bias = 2
    assert lib.lsl_layer_layout_get(C.byref(c), C.byref(_abi.LayerLayout())) == _abi.LSL_ERR_INVALID_ARG
    # a misaligned bias on a weight
    w = _abi.Weight(_abi.WFMT_BF16, 0, 64, 64, None, None, 256, None, None, 258)
    assert lib.lora_linear_fwd(256, 8, C.byref(w), 256, 256, 8, 2.0, 256, 256, None, 0, None) == _abi.LSL_ERR_INVALID_ARG
    # scaling off (NULL or factor 0) is accepted with an empty input
    assert lib.lsl_rope(None, 0, 128, 1, 128, 4, 1e4, None, 0, None) == _abi.LSL_OK


def test_workspace_queries_with_zero_tokens(L):
    """Workspace sizing with no tokens (batch 0 or seq 0) is defined and does not
    divide by an empty tile count."""
    from layer_streamed_lora_amd import _abi
    from layer_streamed_lora_amd import model as M
    from synth.configs import LLAMA8B_LAYER, QWEN05B_LAYER
    lib = L.lib()
    for shape in (LLAMA8B_LAYER, QWEN05B_LAYER):
        cfg = M.layer_cfg(shape)
        for batch, seq in ((0, 16), (4, 0), (0, 0)):
            for mode in (_abi.MODE_FWD, _abi.MODE_BWD):
                assert lib.lsl_layer_workspace_bytes(C.byref(cfg), batch, seq, mode) >= 0
    assert lib.lsl_ce_workspace_bytes(0, 4096, 128256) > 0
    assert L.lora_linear_workspace_bytes(0, 4096, 4096, 16) >= 0
    assert lib.lsl_attention_workspace_bytes(0, 0, 32, 8, 128) >= 0


def test_attention_workspace_holds_the_balanced_dkv_scratch(L):
    """The backward's workspace: the float32 row sums [batch x n_q x seq], and,
    when the key tiles are few (batch x n_kv x ceil(seq / 32) <= 512, where the
    dK/dV work is spread evenly over the workgroups), 256-byte-aligned arrival
    counts (one per key tile) and 2 ceil(seq / 32) - 1 float32 partial slots of
    2 x 32 x head_dim per (sequence, kv head)."""
    lib = L.lib()
    rows = 1 * 32 * 1024 * 4
    cnt = 256 * ((8 * 32 * 4 + 255) // 256)
    part = 8 * 63 * (2 * 32 * 128) * 4
    assert lib.lsl_attention_workspace_bytes(1, 1024, 32, 8, 128) == rows + cnt + part
    # 3 x 8 x 32 = 768 key tiles: one workgroup per key tile, row sums only
    assert lib.lsl_attention_workspace_bytes(3, 1024, 8, 8, 128) == 3 * 8 * 1024 * 4
    # a single key tile needs no balancing
    assert lib.lsl_attention_workspace_bytes(1, 32, 4, 2, 64) == 256 * ((4 * 32 * 4 + 255) // 256)


def test_size_limits_rejected_before_any_launch(L):
    """Shapes past the 32-bit buffer-offset limits are rejected by every entry
    point before its first launch (these calls would fail on any launch here,
    where there is no GPU): the LoRA linear's side product and GEMM, the
    cross-entropy's lm_head GEMM (ahead of its label count), and a decoder
    layer whose down-projection GEMM is the first to exceed the limit."""
    from layer_streamed_lora_amd import _abi
    from layer_streamed_lora_amd import model as M
    from synth.configs import LLAMA8B_LAYER
    lib = L.lib()
    big = 1 << 62
    T = 1 << 20  # (T + 64) x 2048 bf16 activations exceed 4 GiB
    w = _abi.Weight(_abi.WFMT_BF16, 0, 64, 2048, None, None, 256)
    assert lib.lora_linear_fwd(256, T, C.byref(w), 256, 256, 8, 2.0, 256, 256, 256, big, None) == \
        _abi.LSL_ERR_UNSUPPORTED
    assert b"4 GiB" in lib.lsl_last_error()
    # the backward's u = dy B reads dy [T x n_out]: n_out 2048 exceeds the limit
    w2 = _abi.Weight(_abi.WFMT_BF16, 0, 2048, 64, None, None, 256)
    assert lib.lora_linear_bwd(256, 256, 256, T, C.byref(w2), 256, 256, 8, 2.0, 256, 256, 256, 256, big, None) == \
        _abi.LSL_ERR_UNSUPPORTED
    # vocabulary 2^21 x hidden 1024 bf16 head: (V + 128) H 2 bytes > 4 GiB; ce_check allows it
    V, H = 1 << 21, 1024
    assert lib.fused_ce_loss_fwd(256, 256, 256, 64, H, V, -100, 256, 256, 256, big, None) == _abi.LSL_ERR_UNSUPPORTED
    assert b"4 GiB" in lib.lsl_last_error()
    # the backward works per 32768-column chunk, so that head is fine there; its
    # gradient chunk G [T x 32768] bf16 exceeds the limit from T = 65280 tokens
    assert lib.fused_ce_loss_bwd(256, 256, 256, 256, 70000, 64, 65536, -100, 1.0, 256, 256, big, None) == \
        _abi.LSL_ERR_UNSUPPORTED
    assert lib.fused_ce_logprobs(256, 256, 256, 64, H, V, -100, 1, 256, 256, 256, big, None) == _abi.LSL_ERR_UNSUPPORTED
    # one Llama-8B layer over 160000 tokens: the inter-wide operands exceed 4 GiB
    cfg = M.layer_cfg(LLAMA8B_LAYER)
    lo = _abi.LoraSet((C.c_void_p * 4)(*[256] * 4), (C.c_void_p * 4)(*[256] * 4))
    gr = _abi.LoraGrads((C.c_void_p * 4)(*[256] * 4), (C.c_void_p * 4)(*[256] * 4))
    assert lib.decoder_layer_fwd(C.byref(cfg), 256, C.byref(lo), 256, 1, 160000, 256, None, 256, big, None) == \
        _abi.LSL_ERR_UNSUPPORTED
    assert b"4 GiB" in lib.lsl_last_error()
    assert lib.decoder_layer_bwd(C.byref(cfg), 256, C.byref(lo), 256, 256, 1, 160000, 256, C.byref(gr), None, 256,
                                 big, None) == _abi.LSL_ERR_UNSUPPORTED
    # a t_keep buffer must be 256-byte aligned (checked before anything else is looked at)
    assert lib.decoder_layer_fwd(C.byref(cfg), 256, C.byref(lo), 256, 1, 16, 256, 272, 256, big, None) == \
        _abi.LSL_ERR_INVALID_ARG
    assert b"t_keep" in lib.lsl_last_error()
    assert lib.decoder_layer_bwd(C.byref(cfg), 256, C.byref(lo), 256, 256, 1, 16, 256, C.byref(gr), 272, 256,
                                 big, None) == _abi.LSL_ERR_INVALID_ARG
    # its size: the four projections' products [T x 3r | r | 2r | r] bf16, regions 256-byte aligned
    T, r = 300, LLAMA8B_LAYER.lora_r
    assert M.layer_tkeep_bytes(cfg, 1, T) == sum((T * k * r * 2 + 255) // 256 * 256 for k in (3, 1, 2, 1))


@pytest.mark.parametrize("mode", [0, 1])
def test_layer_workspace_map_regions(L, mode):
    """The layer's intermediates sit in 256-byte aligned, disjoint regions of
    their sizes inside the workspace; the backward entries are 0 in the
    forward mode."""
    from layer_streamed_lora_amd import _abi
    from layer_streamed_lora_amd import model as M
    from synth.configs import LLAMA8B_LAYER
    s = LLAMA8B_LAYER
    batch, seq = 2, 300
    T, H, I, r, Q, KV = batch * seq, s.hidden, s.inter, s.lora_r, s.q_dim, s.kv_dim
    NQKV = Q + 2 * KV
    cfg = M.layer_cfg(s)
    m = M.layer_workspace_map(cfg, batch, seq, mode)
    total = M.layer_workspace_bytes(cfg, batch, seq, mode)
    size = {"n1": 2 * T * H, "t_qkv": 6 * T * r, "qkv": 2 * T * NQKV, "qk_rope": 2 * T * NQKV, "attn": 2 * T * Q,
            "lse": 4 * batch * s.n_q * seq, "t_o": 2 * T * r, "h1": 2 * T * H, "n2": 2 * T * H, "t_gu": 4 * T * r,
            "gu": 4 * T * I, "act": 2 * T * I, "t_down": 2 * T * r, "u_down": 2 * T * r, "d_act": 2 * T * I,
            "d_gu": 4 * T * I, "u_gu": 4 * T * r, "d_n2": 2 * T * H, "d_h1": 2 * T * H, "u_o": 2 * T * r,
            "d_attn": 2 * T * Q, "d_qk_rope": 2 * T * NQKV, "d_qkv": 2 * T * NQKV, "u_qkv": 6 * T * r,
            "d_n1": 2 * T * H, "attn32": 4 * T * Q}
    bwd = set(_abi.WS_MAP_FIELDS[13:])
    regions = []
    for n in _abi.WS_MAP_FIELDS:
        if mode == _abi.MODE_FWD and n in bwd:
            assert m[n] == 0, n
            continue
        assert m[n] % 256 == 0, n
        regions.append((m[n], size[n], n))
    regions.sort()
    for (o, b, n), (o2, _, n2) in zip(regions, regions[1:]):
        assert o + b <= o2, (n, n2)
    assert regions[-1][0] + regions[-1][1] <= total
    assert lib_status_bad_mode(L, cfg) == _abi.LSL_ERR_INVALID_ARG


def lib_status_bad_mode(L, cfg):
    from layer_streamed_lora_amd import _abi
    out = _abi.LayerWsMap()
    return L.lib().lsl_layer_workspace_map(C.byref(cfg), 1, 16, 2, C.byref(out))
