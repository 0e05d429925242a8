// Entry points declared in lsl.h that are not built yet report UNSUPPORTED.
#include "common.h"
using namespace lsl;
#define LSL_STUB(name) return set_error(LSL_ERR_UNSUPPORTED, name ": not built yet")

extern "C" size_t lsl_ce_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }
extern "C" lsl_status fused_ce_loss_fwd(const uint16_t*, const uint16_t*, const int32_t*, int64_t, int64_t, int64_t,
                                        int32_t, float*, float*, void*, size_t, lsl_stream) { LSL_STUB("fused_ce_loss_fwd"); }
extern "C" lsl_status fused_ce_loss_bwd(const uint16_t*, const uint16_t*, const int32_t*, const float*, int64_t, int64_t,
                                        int64_t, int32_t, float, uint16_t*, void*, size_t, lsl_stream) { LSL_STUB("fused_ce_loss_bwd"); }
