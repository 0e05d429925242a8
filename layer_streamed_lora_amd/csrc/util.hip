// Error reporting, device properties and the ABI version.
#include "common.h"
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

namespace lsl {
static thread_local std::string g_err;

lsl_status set_error(lsl_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

lsl_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(LSL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return LSL_OK;
}
}  // namespace lsl

extern "C" const char* lsl_last_error(void) { return lsl::g_err.c_str(); }
extern "C" int32_t lsl_abi_version(void) { return 3; }

extern "C" lsl_status lsl_device_info(int32_t device, lsl_device_props* out) {
  if (!out) return lsl::set_error(LSL_ERR_INVALID_ARG, "lsl_device_info: out is NULL");
  hipDeviceProp_t p;
  hipError_t e = hipGetDeviceProperties(&p, device);
  if (e != hipSuccess) return lsl::set_error(LSL_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  memset(out, 0, sizeof *out);
  out->cu_count = p.multiProcessorCount;
  out->clock_khz = p.clockRate;
  out->mem_clock_khz = p.memoryClockRate;
  out->mem_bus_bits = p.memoryBusWidth;
  out->hbm_bytes = (int64_t)p.totalGlobalMem;
  out->lds_bytes_per_cu = (int32_t)p.maxSharedMemoryPerMultiProcessor;
  strncpy(out->arch, p.gcnArchName, sizeof(out->arch) - 1);
  return LSL_OK;
}
