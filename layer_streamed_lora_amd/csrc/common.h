// Shared device/host helpers of the HIP library (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LSL_DEV __device__ __forceinline__

// bf16 bits <-> float. Float -> bf16 uses the hardware round-to-nearest-even
// conversion (v_cvt_pk_bf16_f32 on gfx950).
LSL_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
LSL_DEV uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
LSL_DEV uint32_t pack2(float lo, float hi) {
  bf16x2 r; r[0] = (__bf16)lo; r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
LSL_DEV float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
LSL_DEV float hi_bf(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// wave64 reductions
LSL_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
LSL_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Host-side status plumbing shared by every translation unit.
#include "../../include/lsl.h"
namespace lsl {
lsl_status set_error(lsl_status st, const char* fmt, ...);
lsl_status check_launch(const char* what);
inline bool aligned(const void* p, size_t a) { return (((uintptr_t)p) & (a - 1)) == 0; }
}  // namespace lsl
