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

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group,
// lane j passes the address of row (j >> 2), columns 4 (j & 3) .. +3 of a 4 x 16
// block and receives column j of the block, rows 0..3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
LSL_DEV u32x2 ld_tr4(const uint16_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}
// MFMA operand whose reduction index runs down the rows of a row-major LDS tile:
// lane l (g = l >> 4) gets column c0 + l % 16 at rows r0 + 4g + s (slots 0..3)
// and r0 + 16 + 4g + s (slots 4..7) -- the permuted reduction order in which
// two 16-row MFMA results are packed into one operand. The other operand of the
// product must present its reduction index in the same order.
LSL_DEV bf16x8 ld_tr8(const uint16_t* tile, int ld, int r0, int c0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* p = tile + (r0 + 4 * g + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const u32x2 x = ld_tr4(p), y = ld_tr4(p + 16 * ld);
  return __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
}

// Fixed-order reductions across workgroups without a second kernel. The
// workgroups that share an output tile store float32 partials with
// device-coherent stores (wt_store4: the sc1 cache policy, the one the gfx942
// memory model gives device-scope atomic stores, which write through the XCD's
// L2), then call last_arrival. It returns true (in every thread) in the
// workgroup that arrives last; that one reads the partials back with
// device-coherent loads (wt_load4, likewise never served from a stale L2 line)
// and adds them in a fixed order, so the bits do not depend on the arrival
// order. The count (zero before the first arrival) is reset for the next
// launch. A device-scope fence would make plain stores visible too, but on this
// chip it writes back and invalidates the XCD's whole L2, and hundreds of
// workgroups fencing at once cost more than the work they hand over.
constexpr int CPOL_SC1 = 16;  // buffer instruction cache-policy bit: sc1 (device scope)
LSL_DEV __amdgpu_buffer_rsrc_t wt_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
LSL_DEV void wt_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, CPOL_SC1);
}
LSL_DEV f32x4 wt_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CPOL_SC1));
}
LSL_DEV bool last_arrival(unsigned* cnt, int S) {
  __shared__ unsigned prev;
  // this thread's partial stores are complete (written through) before the
  // workgroup arrives
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (unsigned)S - 1) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return prev == (unsigned)S - 1;
}

// Host-side status plumbing shared by every translation unit.
#include "../../include/lsl.h"
namespace lsl {
lsl_status set_error(lsl_status st, const char* fmt, ...);
lsl_status check_launch(const char* what);
inline bool aligned(const void* p, size_t a) { return (((uintptr_t)p) & (a - 1)) == 0; }
}  // namespace lsl
