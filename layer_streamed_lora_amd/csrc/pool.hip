// Two-slot (n-slot) HBM layer pool fed from a pinned host store.
//
// The pages keep the frozen base in page-locked host memory and give the GPU a
// pair of layer-sized VRAM buffers ("Soup: ...", section "Layer Streaming: The
// Mechanism Behind the 4 GB Claim"). Here each slot is filled by one
// hipMemcpyAsync on a dedicated copy stream (the DMA engine), and the two
// streams are ordered by events only:
//   load:    copy stream waits for the slot's `free` event (its previous user
//            finished), copies, records `ready`;
//   acquire: compute stream waits for `ready`;
//   release: compute stream records `free`.
// So compute on one slot overlaps the copy into the other, and no host thread
// ever blocks. The state machine below rejects out-of-order use (STATE) before
// anything is enqueued.
//
// Poison mode (LSL_POISON_SLOTS set to a non-zero value when the pool is
// created): every load first fills the whole slot with 0xFF bytes on the copy
// stream, after the wait for the slot's release and before the copy. A bf16
// 0xFFFF is a NaN and an NF4 absmax of 0xFFFFFFFF too, so a kernel that reads
// a slot outside its load/acquire/release window, or past the layer's bytes,
// poisons its results instead of silently reading a stale layer: the pages
// stress that streaming failures are silent ("Exact Layer Streaming ...",
// abstract).
#include "common.h"
#include "api_util.h"
#include <cstdlib>
#include <cstring>
#include <vector>

enum SlotState { SLOT_EMPTY = 0, SLOT_LOADED = 1, SLOT_ACQUIRED = 2, SLOT_RELEASED = 3 };

struct lsl_pool {
  int n = 0;
  size_t slot_bytes = 0;
  hipStream_t copy = nullptr;
  std::vector<void*> ptr;
  std::vector<hipEvent_t> ready, freed;
  std::vector<int> state;
  std::vector<bool> free_recorded;
  bool poison = false;
  // optional copy statistics
  std::vector<hipEvent_t> st_start, st_end;
  std::vector<size_t> st_bytes;
  int st_count = 0;
};

using namespace lsl;

static lsl_status hip_fail(const char* what, hipError_t e) {
  return set_error(LSL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

extern "C" lsl_status lsl_pool_create(lsl_pool** out, void* const* slot_ptrs, int32_t n_slots, size_t slot_bytes,
                                      lsl_stream copy_stream) {
  if (!out || !slot_ptrs || n_slots < 1 || n_slots > 16 || slot_bytes == 0)
    return set_error(LSL_ERR_INVALID_ARG, "lsl_pool_create: bad arguments");
  for (int i = 0; i < n_slots; ++i)
    if (!slot_ptrs[i] || !aligned(slot_ptrs[i], 256))
      return set_error(LSL_ERR_INVALID_ARG, "lsl_pool_create: slot %d pointer NULL or not 256-byte aligned", i);
  lsl_pool* p = new lsl_pool();
  p->n = n_slots;
  p->slot_bytes = slot_bytes;
  p->copy = (hipStream_t)copy_stream;
  p->ptr.assign(slot_ptrs, slot_ptrs + n_slots);
  p->ready.assign(n_slots, nullptr);
  p->freed.assign(n_slots, nullptr);
  p->state.assign(n_slots, SLOT_EMPTY);
  p->free_recorded.assign(n_slots, false);
  if (const char* e = getenv("LSL_POISON_SLOTS")) p->poison = e[0] != '\0' && strcmp(e, "0") != 0;
  for (int i = 0; i < n_slots; ++i) {
    hipError_t e;
    // ordering only: no timestamps on the per-layer events (statistics use their own)
    if ((e = hipEventCreateWithFlags(&p->ready[i], hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&p->freed[i], hipEventDisableTiming)) != hipSuccess) {
      lsl_pool_destroy(p);
      return hip_fail("lsl_pool_create: hipEventCreate", e);
    }
  }
  *out = p;
  return LSL_OK;
}

static void stats_free(lsl_pool* p) {
  for (auto e : p->st_start) (void)hipEventDestroy(e);
  for (auto e : p->st_end) (void)hipEventDestroy(e);
  p->st_start.clear();
  p->st_end.clear();
  p->st_bytes.clear();
  p->st_count = 0;
}

extern "C" lsl_status lsl_pool_destroy(lsl_pool* p) {
  if (!p) return LSL_OK;
  for (int i = 0; i < p->n; ++i) {
    if (p->ready[i]) (void)hipEventDestroy(p->ready[i]);
    if (p->freed[i]) (void)hipEventDestroy(p->freed[i]);
  }
  stats_free(p);
  delete p;
  return LSL_OK;
}

extern "C" lsl_status lsl_pool_stats_enable(lsl_pool* p, int32_t max_loads) {
  if (!p || max_loads < 0 || max_loads > (1 << 20))
    return set_error(LSL_ERR_INVALID_ARG, "lsl_pool_stats_enable: bad arguments");
  stats_free(p);
  p->st_start.assign(max_loads, nullptr);
  p->st_end.assign(max_loads, nullptr);
  p->st_bytes.assign(max_loads, 0);
  for (int i = 0; i < max_loads; ++i) {
    hipError_t e;
    if ((e = hipEventCreate(&p->st_start[i])) != hipSuccess || (e = hipEventCreate(&p->st_end[i])) != hipSuccess) {
      stats_free(p);
      return hip_fail("lsl_pool_stats_enable: hipEventCreate", e);
    }
  }
  return LSL_OK;
}

extern "C" lsl_status lsl_pool_stats_read(lsl_pool* p, int32_t* loads, double* bytes, double* seconds) {
  if (!p || !loads || !bytes || !seconds) return set_error(LSL_ERR_INVALID_ARG, "lsl_pool_stats_read: NULL argument");
  double b = 0.0, s = 0.0;
  for (int i = 0; i < p->st_count; ++i) {
    hipError_t e = hipEventSynchronize(p->st_end[i]);
    if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, p->st_start[i], p->st_end[i])) != hipSuccess) return hip_fail("hipEventElapsedTime", e);
    s += ms * 1e-3;
    b += (double)p->st_bytes[i];
  }
  *loads = p->st_count;
  *bytes = b;
  *seconds = s;
  p->st_count = 0;
  return LSL_OK;
}

static lsl_status check_slot(lsl_pool* p, int32_t slot, const char* fn) {
  if (!p) return set_error(LSL_ERR_INVALID_ARG, "%s: pool is NULL", fn);
  if (slot < 0 || slot >= p->n) return set_error(LSL_ERR_INVALID_ARG, "%s: slot %d out of range [0, %d)", fn, slot, p->n);
  return LSL_OK;
}

extern "C" lsl_status load_layer_async(lsl_pool* p, int32_t slot, const void* host_ptr, size_t bytes) {
  const char* fn = "load_layer_async";
  LSL_TRY(check_slot(p, slot, fn));
  if (!host_ptr || bytes == 0 || bytes > p->slot_bytes)
    return set_error(LSL_ERR_INVALID_ARG, "%s: host pointer NULL or size %zu not in (0, %zu]", fn, bytes, p->slot_bytes);
  if (p->state[slot] == SLOT_LOADED || p->state[slot] == SLOT_ACQUIRED)
    return set_error(LSL_ERR_STATE, "%s: slot %d is still %s", fn, slot,
                     p->state[slot] == SLOT_LOADED ? "loaded and not yet used" : "acquired");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, host_ptr);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return set_error(LSL_ERR_NOT_PINNED, "%s: host pointer is not page-locked host memory", fn);
  }
  if (p->free_recorded[slot] && (e = hipStreamWaitEvent(p->copy, p->freed[slot], 0)) != hipSuccess)
    return hip_fail("load_layer_async: hipStreamWaitEvent", e);
  if (p->poison && (e = hipMemsetAsync(p->ptr[slot], 0xFF, p->slot_bytes, p->copy)) != hipSuccess)
    return hip_fail("load_layer_async: hipMemsetAsync (poison)", e);
  const bool stat = p->st_count < (int)p->st_start.size();
  if (stat && (e = hipEventRecord(p->st_start[p->st_count], p->copy)) != hipSuccess) return hip_fail("hipEventRecord", e);
  if ((e = hipMemcpyAsync(p->ptr[slot], host_ptr, bytes, hipMemcpyHostToDevice, p->copy)) != hipSuccess)
    return hip_fail("load_layer_async: hipMemcpyAsync", e);
  if ((e = hipEventRecord(p->ready[slot], p->copy)) != hipSuccess) return hip_fail("hipEventRecord", e);
  if (stat) {
    if ((e = hipEventRecord(p->st_end[p->st_count], p->copy)) != hipSuccess) return hip_fail("hipEventRecord", e);
    p->st_bytes[p->st_count++] = bytes;
  }
  p->state[slot] = SLOT_LOADED;
  return LSL_OK;
}

extern "C" lsl_status lsl_pool_acquire(lsl_pool* p, int32_t slot, lsl_stream compute, void** slot_ptr) {
  const char* fn = "lsl_pool_acquire";
  LSL_TRY(check_slot(p, slot, fn));
  if (p->state[slot] != SLOT_LOADED)
    return set_error(LSL_ERR_STATE, "%s: slot %d has no pending load (state %d)", fn, slot, p->state[slot]);
  hipError_t e = hipStreamWaitEvent((hipStream_t)compute, p->ready[slot], 0);
  if (e != hipSuccess) return hip_fail("lsl_pool_acquire: hipStreamWaitEvent", e);
  p->state[slot] = SLOT_ACQUIRED;
  if (slot_ptr) *slot_ptr = p->ptr[slot];
  return LSL_OK;
}

extern "C" lsl_status lsl_pool_release(lsl_pool* p, int32_t slot, lsl_stream compute) {
  const char* fn = "lsl_pool_release";
  LSL_TRY(check_slot(p, slot, fn));
  if (p->state[slot] != SLOT_ACQUIRED)
    return set_error(LSL_ERR_STATE, "%s: slot %d is not acquired (state %d)", fn, slot, p->state[slot]);
  hipError_t e = hipEventRecord(p->freed[slot], (hipStream_t)compute);
  if (e != hipSuccess) return hip_fail("lsl_pool_release: hipEventRecord", e);
  p->free_recorded[slot] = true;
  p->state[slot] = SLOT_RELEASED;
  return LSL_OK;
}

extern "C" lsl_status lsl_pool_reuse(lsl_pool* p, int32_t slot) {
  const char* fn = "lsl_pool_reuse";
  LSL_TRY(check_slot(p, slot, fn));
  if (p->state[slot] != SLOT_RELEASED)
    return set_error(LSL_ERR_STATE, "%s: slot %d holds no released layer (state %d)", fn, slot, p->state[slot]);
  p->state[slot] = SLOT_LOADED;
  return LSL_OK;
}
