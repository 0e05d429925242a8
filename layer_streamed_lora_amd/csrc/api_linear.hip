// C-ABI entry points of the LoRA linear and of the standalone support ops.
// Every entry validates all arguments before enqueueing anything.
#include "common.h"
#include "gemm.h"
#include "small.h"
#include "api_util.h"
#include <mutex>

// bytes of the allocation-free forward's scratch: 88 MiB, the largest forward
// partials of a Llama-3.1-8B projection up to 1024 tokens (q|k|v just below 1024
// tokens: 351 stream-K slots of 256 KiB; from 1024 tokens the split partials
// of o and down, four of 1024 x 4096 floats, take 64 MiB), plus 64 KiB for the
// arrival counts
#ifndef LSL_NOALLOC_SCRATCH_BYTES
#define LSL_NOALLOC_SCRATCH_BYTES ((88u << 20) + (64u << 10))
#endif

using namespace lsl;

namespace lsl {

bool lora_rank_ok(int32_t r) { return r >= 8 && r <= 64 && r % 8 == 0; }

// Workspace of the LoRA linear: the arrival counts of the side products and of
// the GEMM (zeroed at the start of each call), then (bwd) u = dy B [T x r] bf16,
// then one region reused in turn by the side products' partials and the GEMM's
// split-K / stream-K partials.
static size_t linear_counts(int64_t T, int64_t N, int64_t K) {
  return std::max({lora_counts_needed(T, std::max(N, K)), gemm_counts_needed(T, N, K), gemm_counts_needed(T, K, N)});
}
static size_t linear_counts_bytes(int64_t T, int64_t N, int64_t K) {
  return align256(linear_counts(T, N, K) * sizeof(unsigned));
}

size_t linear_ws_fwd(int64_t T, int64_t N, int64_t K, int r) {
  return linear_counts_bytes(T, N, K) + std::max(lora_nt_ws_bytes(T, K, r), gemm_split_bytes(T, N, K));
}

size_t linear_ws_bwd(int64_t T, int64_t N, int64_t K, int r) {
  size_t part = lora_nt_ws_bytes(T, N, r);
  part = std::max(part, gemm_split_bytes(T, K, N));
  part = std::max(part, lora_tn_ws_bytes(T, K, r));
  part = std::max(part, lora_tn_ws_bytes(T, N, r));
  return linear_counts_bytes(T, N, K) + align256((size_t)T * r * 2) + part;
}

static lsl_status check_weight(const lsl_weight* W, const char* fn) {
  if (!W) return set_error(LSL_ERR_INVALID_ARG, "%s: W is NULL", fn);
  if (W->n_out <= 0 || W->k_in <= 0 || W->k_in % 64 || W->n_out % 64)
    return set_error(LSL_ERR_UNSUPPORTED, "%s: weight [%lld x %lld] needs k_in and n_out multiples of 64", fn,
                     (long long)W->n_out, (long long)W->k_in);
  if (W->fmt == LSL_WFMT_NF4) {
    if (!W->nf4 || !W->absmax || W->bf16 || W->absmax_q || W->absmax_scale || !aligned(W->nf4, 16) ||
        !aligned(W->absmax, 4))
      return set_error(LSL_ERR_INVALID_ARG, "%s: NF4 weight needs 16-byte aligned codes and absmax, bf16 NULL", fn);
  } else if (W->fmt == LSL_WFMT_NF4DQ) {
    if (!W->nf4 || !W->absmax_q || !W->absmax_scale || W->absmax || W->bf16 || !aligned(W->nf4, 16) ||
        !aligned(W->absmax_scale, 4))
      return set_error(LSL_ERR_INVALID_ARG,
                       "%s: NF4DQ weight needs 16-byte aligned codes, absmax_q and absmax_scale; absmax, bf16 NULL", fn);
  } else if (W->fmt == LSL_WFMT_BF16) {
    if (!W->bf16 || W->nf4 || W->absmax || W->absmax_q || W->absmax_scale || !aligned(W->bf16, 16))
      return set_error(LSL_ERR_INVALID_ARG, "%s: bf16 weight needs a 16-byte aligned pointer, NF4 pointers NULL", fn);
  } else {
    return set_error(LSL_ERR_INVALID_ARG, "%s: unknown weight format %d", fn, W->fmt);
  }
  if (W->bias && !aligned(W->bias, 16)) return set_error(LSL_ERR_INVALID_ARG, "%s: bias not 16-byte aligned", fn);
  return LSL_OK;
}

static void weight_into(GemmDesc& g, const lsl_weight* W) {
  g.wfmt = W->fmt;
  g.wb = W->bf16; g.wq = W->nf4; g.wa = W->absmax; g.wq8 = W->absmax_q; g.wsc = W->absmax_scale;
}

}  // namespace lsl

extern "C" size_t lsl_lora_linear_bwd_u_offset(int64_t T, int64_t n_out, int64_t k_in) {
  return T > 0 && n_out > 0 && k_in > 0 ? linear_counts_bytes(T, n_out, k_in) : 0;
}

extern "C" size_t lsl_lora_linear_workspace_bytes(int64_t T, int64_t n_out, int64_t k_in, int32_t r) {
  if (T < 0 || n_out <= 0 || k_in <= 0 || !lora_rank_ok(r)) return 0;
  return std::max(linear_ws_fwd(T, n_out, k_in, r), linear_ws_bwd(T, n_out, k_in, r));
}

extern "C" lsl_status lora_linear_fwd(const uint16_t* x, int64_t T, const lsl_weight* W, const uint16_t* A,
                                      const uint16_t* B, int32_t r, float scale, uint16_t* y, uint16_t* t_out,
                                      void* ws, size_t ws_bytes, lsl_stream stream) {
  const char* fn = "lora_linear_fwd";
  LSL_TRY(check_weight(W, fn));
  if (T < 0) return set_error(LSL_ERR_INVALID_ARG, "%s: T < 0", fn);
  if (!lora_rank_ok(r)) return set_error(LSL_ERR_UNSUPPORTED, "%s: rank %d must be a multiple of 8 in [8, 64]", fn, r);
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {x, A, B, y, t_out}));
  const size_t need = linear_ws_fwd(T, W->n_out, W->k_in, r);
  if (ws_bytes < need || !ws || !aligned(ws, 256))
    return set_error(LSL_ERR_WORKSPACE, "%s: workspace %zu < %zu (or not 256-byte aligned)", fn, ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  const size_t ncnt = linear_counts(T, W->n_out, W->k_in);
  unsigned* cnt = (unsigned*)ws;
  float* part = (float*)((char*)ws + linear_counts_bytes(T, W->n_out, W->k_in));
  LoraNt nt;
  nt.p = x; nt.ldp = W->k_in; nt.T = T; nt.K = W->k_in; nt.kl = r; nt.a_full = A;
  nt.out = t_out; nt.ldo = r; nt.ws = part; nt.cnt = cnt;
  GemmDesc g;
  g.x = x; g.ldx = W->k_in; weight_into(g, W); g.kn = false;
  g.M = T; g.N = W->n_out; g.K = W->k_in;
  g.lora = 1; g.la = t_out; g.ldla = r; g.kl = r; g.lb = B; g.r = r; g.nseg = 1; g.seg_end[0] = W->n_out;
  g.scale = scale; g.y = y; g.ldy = W->n_out; g.split_ws = part; g.cnt = cnt; g.bias = W->bias;
  // every launch's conditions first, so that a rejected call enqueues nothing
  LSL_TRY(lora_nt_check(nt));
  LSL_TRY(gemm_check(g));
  LSL_TRY(lora_counts_zero(cnt, ncnt, s));
  LSL_TRY(lora_nt_launch(nt, s));
  return gemm_launch(g, s);
}

extern "C" lsl_status lora_linear_bwd(const uint16_t* x, const uint16_t* t, const uint16_t* dy, int64_t T,
                                      const lsl_weight* W, const uint16_t* A, const uint16_t* B, int32_t r,
                                      float scale, uint16_t* dx, float* dA, float* dB, void* ws, size_t ws_bytes,
                                      lsl_stream stream) {
  const char* fn = "lora_linear_bwd";
  LSL_TRY(check_weight(W, fn));
  if (T < 0) return set_error(LSL_ERR_INVALID_ARG, "%s: T < 0", fn);
  if (!lora_rank_ok(r)) return set_error(LSL_ERR_UNSUPPORTED, "%s: rank %d must be a multiple of 8 in [8, 64]", fn, r);
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {x, t, dy, A, B, dA, dB}));
  if (dx && !aligned(dx, 16)) return set_error(LSL_ERR_INVALID_ARG, "%s: dx misaligned", fn);
  size_t need = linear_ws_bwd(T, W->n_out, W->k_in, r);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return set_error(LSL_ERR_WORKSPACE, "%s: workspace %zu < %zu (or not 256-byte aligned)", fn, ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  const int64_t N = W->n_out, K = W->k_in;
  const size_t ncnt = linear_counts(T, N, K);
  unsigned* cnt = (unsigned*)ws;
  uint16_t* u = (uint16_t*)((char*)ws + linear_counts_bytes(T, N, K));
  float* part = (float*)((char*)u + align256((size_t)T * r * 2));
  LoraNt nt;
  nt.p = dy; nt.ldp = N; nt.T = T; nt.K = N; nt.kl = r; nt.b_full = B; nt.r = r; nt.nseg = 1; nt.seg_end[0] = N;
  nt.out = u; nt.ldo = r; nt.ws = part; nt.cnt = cnt;
  GemmDesc g;
  g.x = dy; g.ldx = N; weight_into(g, W); g.kn = true;
  g.M = T; g.N = K; g.K = N;
  g.lora = 2; g.la = u; g.ldla = r; g.kl = r; g.lb = A; g.r = r;
  g.scale = scale; g.y = dx; g.ldy = K; g.split_ws = part; g.cnt = cnt;
  LoraTn ta;
  ta.p = x; ta.ldp = K; ta.q = u; ta.ldq = r; ta.T = T; ta.W = K; ta.kl = r; ta.scale = scale; ta.dA = dA; ta.ws = part;
  ta.cnt = cnt;
  LoraTn tb;
  tb.p = dy; tb.ldp = N; tb.q = t; tb.ldq = r; tb.T = T; tb.W = N; tb.kl = r; tb.scale = scale; tb.dB = dB;
  tb.r = r; tb.nseg = 1; tb.seg_end[0] = N; tb.ws = part; tb.cnt = cnt;
  // every launch's conditions first, so that a rejected call enqueues nothing
  LSL_TRY(lora_nt_check(nt));
  if (dx) LSL_TRY(gemm_check(g));
  LSL_TRY(lora_tn_check(ta));
  LSL_TRY(lora_tn_check(tb));
  LSL_TRY(lora_counts_zero(cnt, ncnt, s));
  LSL_TRY(lora_nt_launch(nt, s));
  if (dx) LSL_TRY(gemm_launch(g, s));
  LSL_TRY(lora_tn_launch(ta, s));
  return lora_tn_launch(tb, s);
}

// ---------------------------------------------------------------- allocation-free forward
// lora_linear_fwd_noalloc: the same launches as lora_linear_fwd with the
// workspace in a file-scope device array of LSL_NOALLOC_SCRATCH_BYTES (each GPU
// the library runs on holds its own copy until the process ends). Host code
// never passes the array's name to a kernel: its address on the current device
// comes from hipGetSymbolAddress, looked up once per device on the first call.
namespace lsl {
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)LSL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[MAX_DEVICES];

static lsl_status scratch_on_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(LSL_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return set_error(LSL_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return set_error(LSL_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LSL_OK;
}
}  // namespace lsl

extern "C" size_t lsl_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

extern "C" lsl_status lora_linear_fwd_noalloc(const uint16_t* x, int64_t T, const lsl_weight* W, const uint16_t* A,
                                              const uint16_t* B, int32_t r, float scale, uint16_t* y,
                                              uint16_t* t_out, lsl_stream stream) {
  const char* fn = "lora_linear_fwd_noalloc";
  LSL_TRY(check_weight(W, fn));
  if (T < 0) return set_error(LSL_ERR_INVALID_ARG, "%s: T < 0", fn);
  if (!lora_rank_ok(r)) return set_error(LSL_ERR_UNSUPPORTED, "%s: rank %d must be a multiple of 8 in [8, 64]", fn, r);
  if (T == 0) return LSL_OK;
  const size_t need = linear_ws_fwd(T, W->n_out, W->k_in, r);
  if (need > NOALLOC_SCRATCH_BYTES)
    return set_error(LSL_ERR_WORKSPACE, "%s: this shape needs %zu bytes of scratch, more than the %zu the library holds",
                     fn, need, NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  LSL_TRY(scratch_on_current_device(fn, &ws));
  // the side product's arrival counts, which must start at zero, are zeroed by
  // lora_linear_fwd at its start; its split partials are written in full
  // before they are read
  return lora_linear_fwd(x, T, W, A, B, r, scale, y, t_out, ws, NOALLOC_SCRATCH_BYTES, stream);
}

// ---------------------------------------------------------------- support ops
extern "C" lsl_status lsl_rmsnorm_fwd(const uint16_t* x, const uint16_t* w, int64_t T, int64_t H, float eps,
                                      uint16_t* y, lsl_stream stream) {
  const char* fn = "lsl_rmsnorm_fwd";
  if (T < 0 || H <= 0 || H % 8) return set_error(LSL_ERR_INVALID_ARG, "%s: bad sizes (H %% 8 == 0)", fn);
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {x, w, y}));
  return rmsnorm_fwd_launch(x, w, T, H, eps, y, (hipStream_t)stream);
}

extern "C" lsl_status lsl_rmsnorm_bwd(const uint16_t* x, const uint16_t* w, const uint16_t* dy, const uint16_t* dres,
                                      int64_t T, int64_t H, float eps, uint16_t* dx, lsl_stream stream) {
  const char* fn = "lsl_rmsnorm_bwd";
  if (T < 0 || H <= 0 || H % 8) return set_error(LSL_ERR_INVALID_ARG, "%s: bad sizes (H %% 8 == 0)", fn);
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {x, w, dy, dx}));
  if (dres && !aligned(dres, 16)) return set_error(LSL_ERR_INVALID_ARG, "%s: dres misaligned", fn);
  return rmsnorm_bwd_launch(x, w, dy, dres, T, H, eps, dx, (hipStream_t)stream);
}

extern "C" lsl_status lsl_rope(uint16_t* x, int64_t T, int64_t ld, int32_t n_heads, int32_t head_dim, int32_t seq,
                               float theta, const lsl_rope_scaling* scaling, int32_t inverse, lsl_stream stream) {
  const char* fn = "lsl_rope";
  if (T < 0 || n_heads <= 0 || head_dim <= 0 || head_dim % 2 || seq <= 0 || ld < (int64_t)n_heads * head_dim ||
      !(theta > 0.f))
    return set_error(LSL_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (head_dim % 8 || head_dim > 128 || ld % 4)
    return set_error(LSL_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 8 up to 128 and ld of 4", fn);
  LSL_TRY(check_rope_scaling(fn, scaling));
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {x}));
  return rope_launch(x, x, T, ld, n_heads, head_dim, seq, theta, scaling, inverse, (hipStream_t)stream);
}

extern "C" lsl_status lsl_swiglu_fwd(const uint16_t* gu, int64_t T, int64_t I, uint16_t* a, lsl_stream stream) {
  const char* fn = "lsl_swiglu_fwd";
  if (T < 0 || I <= 0 || I % 8) return set_error(LSL_ERR_INVALID_ARG, "%s: bad sizes (I %% 8 == 0)", fn);
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {gu, a}));
  return swiglu_fwd_launch(gu, T, I, a, (hipStream_t)stream);
}

extern "C" lsl_status lsl_swiglu_bwd(const uint16_t* gu, const uint16_t* da, int64_t T, int64_t I, uint16_t* dgu,
                                     lsl_stream stream) {
  const char* fn = "lsl_swiglu_bwd";
  if (T < 0 || I <= 0 || I % 8) return set_error(LSL_ERR_INVALID_ARG, "%s: bad sizes (I %% 8 == 0)", fn);
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {gu, da, dgu}));
  return swiglu_bwd_launch(gu, da, T, I, dgu, (hipStream_t)stream);
}
