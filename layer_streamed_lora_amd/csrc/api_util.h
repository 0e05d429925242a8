// Validation helpers shared by the C-ABI translation units.
#pragma once
#include "common.h"
#include <algorithm>
#include <initializer_list>

#define LSL_TRY(expr)                         \
  do {                                        \
    lsl_status _st = (expr);                  \
    if (_st != LSL_OK) return _st;            \
  } while (0)

namespace lsl {
inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
inline lsl_status check_ptrs(const char* fn, std::initializer_list<const void*> ps, size_t align = 16) {
  int i = 0;
  for (const void* p : ps) {
    if (!p) return set_error(LSL_ERR_INVALID_ARG, "%s: pointer argument %d is NULL", fn, i);
    if (!aligned(p, align))
      return set_error(LSL_ERR_INVALID_ARG, "%s: pointer argument %d is not %zu-byte aligned", fn, i, align);
    ++i;
  }
  return LSL_OK;
}
bool lora_rank_ok(int32_t r);
// NULL or factor 0: no scaling; otherwise factor >= 1, 0 < low < high, original > 0
inline lsl_status check_rope_scaling(const char* fn, const lsl_rope_scaling* sc) {
  if (!sc || sc->factor == 0.f) return LSL_OK;
  if (!(sc->factor >= 1.f) || !(sc->low_freq_factor > 0.f) || !(sc->high_freq_factor > sc->low_freq_factor) ||
      !(sc->original_max_position > 0.f))
    return set_error(LSL_ERR_INVALID_ARG, "%s: bad RoPE scaling (factor >= 1, 0 < low < high, original > 0)", fn);
  return LSL_OK;
}
}  // namespace lsl
