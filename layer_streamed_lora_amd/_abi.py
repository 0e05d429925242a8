"""ctypes declarations of the C ABI in include/lsl.h (argument marshalling only)."""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblsl.so")

LSL_OK, LSL_ERR_INVALID_ARG, LSL_ERR_UNSUPPORTED, LSL_ERR_NOT_PINNED, LSL_ERR_WORKSPACE, LSL_ERR_STATE, LSL_ERR_HIP = range(7)
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "NOT_PINNED", 4: "WORKSPACE", 5: "STATE", 6: "HIP"}
WFMT_NF4, WFMT_BF16, WFMT_NF4DQ = 0, 1, 2
M_QKV, M_O, M_GU, M_DOWN = 0, 1, 2, 3
MODE_FWD, MODE_BWD = 0, 1

vp = C.c_void_p
i32, i64, f32, sz = C.c_int32, C.c_int64, C.c_float, C.c_size_t


class Weight(C.Structure):
    _fields_ = [("fmt", i32), ("pad", i32), ("n_out", i64), ("k_in", i64),
                ("nf4", vp), ("absmax", vp), ("bf16", vp), ("absmax_q", vp), ("absmax_scale", vp),
                ("bias", vp)]


class RopeScaling(C.Structure):
    _fields_ = [("factor", f32), ("low_freq_factor", f32), ("high_freq_factor", f32),
                ("original_max_position", f32)]


class LayerCfg(C.Structure):
    _fields_ = [("hidden", i32), ("n_q", i32), ("n_kv", i32), ("head_dim", i32), ("inter", i32),
                ("rms_eps", f32), ("rope_theta", f32), ("wfmt", i32), ("lora_r", i32), ("lora_scale", f32),
                ("qkv_bias", i32), ("rope_scaling", RopeScaling)]


class LayerLayout(C.Structure):
    _fields_ = [("norm1_off", C.c_uint64), ("norm2_off", C.c_uint64), ("w_off", C.c_uint64 * 4),
                ("absmax_off", C.c_uint64 * 4), ("total_bytes", C.c_uint64),
                ("scale_off", C.c_uint64 * 4), ("bias_off", C.c_uint64)]


WS_MAP_FIELDS = ("n1", "t_qkv", "qkv", "qk_rope", "attn", "lse", "t_o", "h1", "n2", "t_gu", "gu", "act", "t_down",
                 "u_down", "d_act", "d_gu", "u_gu", "d_n2", "d_h1", "u_o", "d_attn", "d_qk_rope", "d_qkv", "u_qkv",
                 "d_n1", "attn32")


class LayerWsMap(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in WS_MAP_FIELDS]


class LoraSet(C.Structure):
    _fields_ = [("A", vp * 4), ("B", vp * 4)]


class LoraGrads(C.Structure):
    _fields_ = [("dA", vp * 4), ("dB", vp * 4)]


class DeviceProps(C.Structure):
    _fields_ = [("cu_count", i32), ("clock_khz", i32), ("mem_clock_khz", i32), ("mem_bus_bits", i32),
                ("hbm_bytes", i64), ("lds_bytes_per_cu", i32), ("pad", i32), ("arch", C.c_char * 64)]


PROTOS = {
    "lsl_last_error": (C.c_char_p, []),
    "lsl_abi_version": (i32, []),
    "lsl_device_info": (i32, [i32, C.POINTER(DeviceProps)]),
    "lsl_nf4_codebook": (i32, [C.POINTER(C.c_float)]),
    "lsl_nf4_quantize": (i32, [vp, i64, i64, vp, vp, vp]),
    "lsl_nf4_dequant": (i32, [vp, vp, i64, i64, vp, vp]),
    "lsl_nf4dq_quantize_absmax": (i32, [vp, i64, vp, vp, vp]),
    "lsl_nf4dq_dequant": (i32, [vp, vp, vp, i64, i64, vp, vp]),
    "lsl_lora_linear_workspace_bytes": (sz, [i64, i64, i64, i32]),
    "lsl_lora_linear_bwd_u_offset": (sz, [i64, i64, i64]),
    "lora_linear_fwd": (i32, [vp, i64, C.POINTER(Weight), vp, vp, i32, f32, vp, vp, vp, sz, vp]),
    "lora_linear_bwd": (i32, [vp, vp, vp, i64, C.POINTER(Weight), vp, vp, i32, f32, vp, vp, vp, vp, sz, vp]),
    "lora_linear_fwd_noalloc": (i32, [vp, i64, C.POINTER(Weight), vp, vp, i32, f32, vp, vp, vp]),
    "lsl_noalloc_scratch_bytes": (sz, []),
    "lsl_layer_layout_get": (i32, [C.POINTER(LayerCfg), C.POINTER(LayerLayout)]),
    "lsl_layer_workspace_bytes": (sz, [C.POINTER(LayerCfg), i32, i32, i32]),
    "lsl_layer_workspace_map": (i32, [C.POINTER(LayerCfg), i32, i32, i32, C.POINTER(LayerWsMap)]),
    "lsl_layer_tkeep_bytes": (sz, [C.POINTER(LayerCfg), i32, i32]),
    "decoder_layer_fwd": (i32, [C.POINTER(LayerCfg), vp, C.POINTER(LoraSet), vp, i32, i32, vp, vp, vp, sz, vp]),
    "decoder_layer_bwd": (i32, [C.POINTER(LayerCfg), vp, C.POINTER(LoraSet), vp, vp, i32, i32, vp,
                                C.POINTER(LoraGrads), vp, vp, sz, vp]),
    "lsl_pool_create": (i32, [C.POINTER(vp), C.POINTER(vp), i32, sz, vp]),
    "lsl_pool_destroy": (i32, [vp]),
    "load_layer_async": (i32, [vp, i32, vp, sz]),
    "lsl_pool_acquire": (i32, [vp, i32, vp, C.POINTER(vp)]),
    "lsl_pool_release": (i32, [vp, i32, vp]),
    "lsl_pool_reuse": (i32, [vp, i32]),
    "lsl_pool_stats_enable": (i32, [vp, i32]),
    "lsl_pool_stats_read": (i32, [vp, C.POINTER(i32), C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "lsl_timing_enable": (i32, [i32, i32]),
    "lsl_timing_read": (i32, [C.POINTER(C.c_double), C.POINTER(i32)]),
    "lsl_timing_disable": (i32, []),
    "lsl_ce_workspace_bytes": (sz, [i64, i64, i64]),
    "fused_ce_loss_fwd": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, vp, vp, sz, vp]),
    "fused_ce_loss_bwd": (i32, [vp, vp, vp, vp, i64, i64, i64, i32, f32, vp, vp, sz, vp]),
    "fused_ce_logprobs": (i32, [vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, vp, sz, vp]),
    "lsl_rmsnorm_fwd": (i32, [vp, vp, i64, i64, f32, vp, vp]),
    "lsl_rmsnorm_bwd": (i32, [vp, vp, vp, vp, i64, i64, f32, vp, vp]),
    "lsl_rope": (i32, [vp, i64, i64, i32, i32, i32, f32, C.POINTER(RopeScaling), i32, vp]),
    "lsl_attention_fwd": (i32, [vp, vp, vp, i64, i64, i32, i32, i32, i32, i32, vp, i64, vp, vp, vp]),
    "lsl_attention_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
    "lsl_attention_bwd": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
    "lsl_swiglu_fwd": (i32, [vp, i64, i64, vp, vp]),
    "lsl_swiglu_bwd": (i32, [vp, vp, i64, i64, vp, vp]),
    "lsl_embed_fwd": (i32, [vp, vp, i64, i64, i64, vp, vp]),
    "lsl_adamw_step": (i32, [vp, vp, vp, vp, vp, i64, i32, f32, f32, f32, f32, f32, vp]),
}


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing (run __graft_entry__.build())")
    lib = C.CDLL(path)
    for name, (res, args) in PROTOS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
