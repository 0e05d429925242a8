// Entry points declared in lsl.h that are not built yet report UNSUPPORTED.
#include "common.h"
using namespace lsl;
#define LSL_STUB(name) return set_error(LSL_ERR_UNSUPPORTED, name ": not built yet")

extern "C" size_t lsl_ce_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }
extern "C" lsl_status fused_ce_loss_fwd(const uint16_t*, const uint16_t*, const int32_t*, int64_t, int64_t, int64_t,
                                        int32_t, float*, float*, void*, size_t, lsl_stream) { LSL_STUB("fused_ce_loss_fwd"); }
extern "C" lsl_status fused_ce_loss_bwd(const uint16_t*, const uint16_t*, const int32_t*, const float*, int64_t, int64_t,
                                        int64_t, int32_t, float, uint16_t*, void*, size_t, lsl_stream) { LSL_STUB("fused_ce_loss_bwd"); }
extern "C" lsl_status lsl_attention_fwd(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int32_t,
                                        int32_t, int32_t, int32_t, int32_t, uint16_t*, int64_t, float*, lsl_stream) { LSL_STUB("lsl_attention_fwd"); }
extern "C" size_t lsl_attention_workspace_bytes(int32_t, int32_t, int32_t, int32_t, int32_t) { return 0; }
extern "C" lsl_status lsl_attention_bwd(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                                        const uint16_t*, const float*, int64_t, int64_t, int32_t, int32_t, int32_t,
                                        int32_t, int32_t, uint16_t*, uint16_t*, uint16_t*, void*, size_t, lsl_stream) { LSL_STUB("lsl_attention_bwd"); }
extern "C" lsl_status lsl_layer_layout_get(const lsl_layer_cfg*, lsl_layer_layout*) { LSL_STUB("lsl_layer_layout_get"); }
extern "C" size_t lsl_layer_workspace_bytes(const lsl_layer_cfg*, int32_t, int32_t, int32_t) { return 0; }
extern "C" lsl_status decoder_layer_fwd(const lsl_layer_cfg*, const void*, const lsl_lora_set*, const uint16_t*, int32_t,
                                        int32_t, uint16_t*, void*, size_t, lsl_stream) { LSL_STUB("decoder_layer_fwd"); }
extern "C" lsl_status decoder_layer_bwd(const lsl_layer_cfg*, const void*, const lsl_lora_set*, const uint16_t*,
                                        const uint16_t*, int32_t, int32_t, uint16_t*, const lsl_lora_grads*, void*,
                                        size_t, lsl_stream) { LSL_STUB("decoder_layer_bwd"); }
