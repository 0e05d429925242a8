// NF4 (4-bit NormalFloat, QLoRA section 3) codebook, blockwise-absmax quantiser
// and standalone dequantiser. The GEMMs dequantise inside their operand staging;
// the standalone kernels build the host store and serve as bandwidth probes.
#include "common.h"
#include "nf4.h"
#include <cmath>

namespace lsl {

// Standard normal CDF from the C library's erfc.
static double norm_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

// Phi^-1(p) for p in (0.5, 1): bisection on the CDF (which is monotone), then
// Newton steps; accurate to a few ulp of the CDF evaluation.
static double norm_ppf_upper(double p) {
  double lo = 0.0, hi = 10.0;
  for (int i = 0; i < 200 && hi - lo > 0.0; ++i) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (norm_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  const double inv_sqrt_2pi = 0.3989422804014327;
  for (int i = 0; i < 3; ++i) {
    double f = norm_cdf(x) - p;
    double d = inv_sqrt_2pi * std::exp(-0.5 * x * x);
    x -= f / d;
  }
  return x;
}

// The NormalFloat construction: offset delta = ((1 - 1/30) + (1 - 1/32)) / 2;
// 8 positive quantiles at the first 8 points of a 9-point grid from delta to
// 1/2, 7 negative ones from an 8-point grid, an exact zero; divided by the
// largest; rounded once to float32.
void nf4_codebook_host(float out[16]) {
  const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  double v[16];
  int n = 0;
  const double step9 = (0.5 - delta) / 8.0, step8 = (0.5 - delta) / 7.0;
  double pos[8], neg[7];
  for (int i = 0; i < 8; ++i) pos[i] = norm_ppf_upper((double)i * step9 + delta);
  for (int i = 0; i < 7; ++i) neg[i] = -norm_ppf_upper((double)i * step8 + delta);
  for (int i = 0; i < 7; ++i) v[n++] = neg[i];  // ascending: most negative first
  v[n++] = 0.0;
  for (int i = 7; i >= 0; --i) v[n++] = pos[i];
  const double top = pos[0];
  for (int i = 0; i < 16; ++i) out[i] = (float)(v[i] / top);
}

const Nf4Table& nf4_table() {
  static Nf4Table t = [] {
    Nf4Table r;
    nf4_codebook_host(r.cb);
    for (int i = 0; i < 15; ++i) r.mid[i] = (r.cb[i] + r.cb[i + 1]) * 0.5f;
    r.mid[15] = 0.f;
    return r;
  }();
  return t;
}

// One thread per 64-element block.
__global__ void nf4_quantize_kernel(const uint16_t* __restrict__ w, int64_t nblocks,
                                    uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                    Nf4Table tab) {
  int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(w + b * 64);
  uint32_t raw[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 q = src[i];
    raw[4 * i] = q[0]; raw[4 * i + 1] = q[1]; raw[4 * i + 2] = q[2]; raw[4 * i + 3] = q[3];
  }
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fmaxf(fabsf(lo_bf(raw[i])), fabsf(hi_bf(raw[i]))));
  absmax[b] = am;
  uint32_t outw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float e0 = am > 0.f ? __fdiv_rn(lo_bf(raw[i]), am) : 0.f;  // element 2i
    float e1 = am > 0.f ? __fdiv_rn(hi_bf(raw[i]), am) : 0.f;  // element 2i+1
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int m = 0; m < 15; ++m) { c0 += e0 > tab.mid[m]; c1 += e1 > tab.mid[m]; }
    uint32_t byte = (c0 << 4) | c1;
    outw[i >> 2] |= byte << ((i & 3) * 8);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(codes + b * 32);
  dst[0] = u32x4{outw[0], outw[1], outw[2], outw[3]};
  dst[1] = u32x4{outw[4], outw[5], outw[6], outw[7]};
}

// One thread per 8 elements (4 code bytes -> 16 output bytes).
__global__ void nf4_dequant_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
                                   int64_t n8, uint16_t* __restrict__ w, Nf4Table tab) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  uint32_t c = reinterpret_cast<const uint32_t*>(codes)[i];
  float am = absmax[i >> 3];
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t byte = (c >> (8 * j)) & 0xFF;
    o[j] = pack2(tab.cb[byte >> 4] * am, tab.cb[byte & 15] * am);
  }
  reinterpret_cast<u32x4*>(w)[i] = o;
}

// Double quantisation of the absmax values: one workgroup per block of 256.
__global__ __launch_bounds__(256) void nf4dq_absmax_kernel(const float* __restrict__ absmax, int64_t n,
                                                           uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float a = i < n ? absmax[i] : 0.f;
  float m = wave_max(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(m, 255.0f);
  if (threadIdx.x == 0) scale[blockIdx.x] = s;
  if (i < n) q[i] = s > 0.f ? (uint8_t)fminf(fmaxf(rintf(__fdiv_rn(a, s)), 0.f), 255.f) : (uint8_t)0;
}

// One thread per 8 elements, absmax' = float(q) * s of its 256-block.
__global__ void nf4dq_dequant_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ qa,
                                     const float* __restrict__ scale, int64_t n8, uint16_t* __restrict__ w,
                                     Nf4Table tab) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  uint32_t c = reinterpret_cast<const uint32_t*>(codes)[i];
  const int64_t b = i >> 3;
  const float am = (float)qa[b] * scale[b >> 8];
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t byte = (c >> (8 * j)) & 0xFF;
    o[j] = pack2(tab.cb[byte >> 4] * am, tab.cb[byte & 15] * am);
  }
  reinterpret_cast<u32x4*>(w)[i] = o;
}

}  // namespace lsl

using namespace lsl;

extern "C" lsl_status lsl_nf4dq_quantize_absmax(const float* absmax, int64_t n, uint8_t* q, float* scale,
                                                lsl_stream stream) {
  if (n < 0) return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4dq_quantize_absmax: n < 0");
  if (n == 0) return LSL_OK;
  if (!absmax || !q || !scale || !aligned(absmax, 4) || !aligned(scale, 4))
    return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4dq_quantize_absmax: null or misaligned pointer");
  hipLaunchKernelGGL(nf4dq_absmax_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     absmax, n, q, scale);
  return check_launch("nf4dq_quantize_absmax");
}

extern "C" lsl_status lsl_nf4dq_dequant(const uint8_t* codes, const uint8_t* q, const float* scale, int64_t rows,
                                        int64_t cols, uint16_t* w, lsl_stream stream) {
  if (rows < 0 || cols < 0 || cols % 64)
    return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4dq_dequant: cols must be a multiple of 64");
  if (rows * cols == 0) return LSL_OK;
  if (!w || !codes || !q || !scale || !aligned(w, 16) || !aligned(codes, 16) || !aligned(scale, 4))
    return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4dq_dequant: null or misaligned pointer");
  int64_t n8 = rows * cols / 8;
  hipLaunchKernelGGL(nf4dq_dequant_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     codes, q, scale, n8, w, nf4_table());
  return check_launch("nf4dq_dequant");
}

extern "C" lsl_status lsl_nf4_codebook(float out[16]) {
  if (!out) return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4_codebook: out is NULL");
  const Nf4Table& t = nf4_table();
  for (int i = 0; i < 16; ++i) out[i] = t.cb[i];
  return LSL_OK;
}

extern "C" lsl_status lsl_nf4_quantize(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* codes,
                                       float* absmax, lsl_stream stream) {
  if (rows < 0 || cols < 0 || cols % 64)
    return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4_quantize: cols must be a multiple of 64 (rows=%lld cols=%lld)",
                     (long long)rows, (long long)cols);
  if (rows * cols == 0) return LSL_OK;
  if (!w || !codes || !absmax || !aligned(w, 16) || !aligned(codes, 16) || !aligned(absmax, 4))
    return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4_quantize: null or misaligned pointer");
  int64_t nb = rows * cols / 64;
  hipLaunchKernelGGL(nf4_quantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, w, nb, codes, absmax, nf4_table());
  return check_launch("nf4_quantize");
}

extern "C" lsl_status lsl_nf4_dequant(const uint8_t* codes, const float* absmax, int64_t rows,
                                      int64_t cols, uint16_t* w, lsl_stream stream) {
  if (rows < 0 || cols < 0 || cols % 64)
    return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4_dequant: cols must be a multiple of 64");
  if (rows * cols == 0) return LSL_OK;
  if (!w || !codes || !absmax || !aligned(w, 16) || !aligned(codes, 16) || !aligned(absmax, 4))
    return set_error(LSL_ERR_INVALID_ARG, "lsl_nf4_dequant: null or misaligned pointer");
  int64_t n8 = rows * cols / 8;
  hipLaunchKernelGGL(nf4_dequant_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, codes, absmax, n8, w, nf4_table());
  return check_launch("nf4_dequant");
}
