// HBM-bound steps of the decoder layer: RMSNorm forward/backward, rotary
// embedding, SwiGLU forward/backward, embedding gather and AdamW. One wave per
// row for the row reductions (wave64 shuffles, no LDS), 16-byte accesses.
#include "common.h"
#include "small.h"
#include <cmath>

namespace lsl {

// ---------------------------------------------------------------- RMSNorm
// y = bf16(x * r * w), r = 1 / sqrt(mean(x^2) + eps). One wave per row.
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                          int64_t T, int64_t H, float eps, uint16_t* __restrict__ y) {
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= T) return;
  const uint16_t* xr = x + row * H;
  float ss = 0.f;
  for (int64_t c = lane * 8; c < H; c += 512) {
    u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) { float a = lo_bf(v[j]), b = hi_bf(v[j]); ss += a * a + b * b; }
  }
  ss = wave_sum(ss);
  float r = 1.0f / sqrtf(ss / (float)H + eps);
  for (int64_t c = lane * 8; c < H; c += 512) {
    u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
    u32x4 g = *reinterpret_cast<const u32x4*>(w + c);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack2(lo_bf(v[j]) * r * lo_bf(g[j]), hi_bf(v[j]) * r * hi_bf(g[j]));
    *reinterpret_cast<u32x4*>(y + row * H + c) = o;
  }
}

// dx = bf16(dres + r (w dy - x r^2 sum(x w dy) / H))
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                          const uint16_t* __restrict__ dy, const uint16_t* __restrict__ dres,
                                                          int64_t T, int64_t H, float eps, uint16_t* __restrict__ dx) {
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= T) return;
  const uint16_t* xr = x + row * H;
  const uint16_t* dr = dy + row * H;
  float ss = 0.f, sd = 0.f;
  for (int64_t c = lane * 8; c < H; c += 512) {
    u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
    u32x4 g = *reinterpret_cast<const u32x4*>(w + c);
    u32x4 d = *reinterpret_cast<const u32x4*>(dr + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = lo_bf(v[j]), b = hi_bf(v[j]);
      ss += a * a + b * b;
      sd += a * lo_bf(g[j]) * lo_bf(d[j]) + b * hi_bf(g[j]) * hi_bf(d[j]);
    }
  }
  ss = wave_sum(ss);
  sd = wave_sum(sd);
  float r = 1.0f / sqrtf(ss / (float)H + eps);
  float c2 = r * r * sd / (float)H;
  for (int64_t c = lane * 8; c < H; c += 512) {
    u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
    u32x4 g = *reinterpret_cast<const u32x4*>(w + c);
    u32x4 d = *reinterpret_cast<const u32x4*>(dr + c);
    u32x4 rs = dres ? *reinterpret_cast<const u32x4*>(dres + row * H + c) : u32x4{0, 0, 0, 0};
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float e0 = lo_bf(rs[j]) + r * (lo_bf(g[j]) * lo_bf(d[j]) - lo_bf(v[j]) * c2);
      float e1 = hi_bf(rs[j]) + r * (hi_bf(g[j]) * hi_bf(d[j]) - hi_bf(v[j]) * c2);
      o[j] = pack2(e0, e1);
    }
    *reinterpret_cast<u32x4*>(dx + row * H + c) = o;
  }
}

lsl_status rmsnorm_fwd_launch(const uint16_t* x, const uint16_t* w, int64_t T, int64_t H, float eps, uint16_t* y, hipStream_t s) {
  if (T == 0) return LSL_OK;
  hipLaunchKernelGGL(rmsnorm_fwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, w, T, H, eps, y);
  return check_launch("rmsnorm_fwd");
}
lsl_status rmsnorm_bwd_launch(const uint16_t* x, const uint16_t* w, const uint16_t* dy, const uint16_t* dres,
                              int64_t T, int64_t H, float eps, uint16_t* dx, hipStream_t s) {
  if (T == 0) return LSL_OK;
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, w, dy, dres, T, H, eps, dx);
  return check_launch("rmsnorm_bwd");
}

// ---------------------------------------------------------------- RoPE
// Thread per (row, frequency index i); the inverse frequency theta^(-2i/d)
// (optionally rescaled the Llama-3.1 way), the angle and its sine/cosine are
// evaluated in float64, then every head's pair (i, i + d/2) is rotated in
// float32 and rounded to bf16 in place.
struct RopeScale {
  double factor, low, high, orig;  // factor 0: none
};

LSL_DEV double rope_inv_freq(int i, int head_dim, double theta, const RopeScale& sc) {
  const double f = pow(theta, -2.0 * (double)i / (double)head_dim);
  if (sc.factor == 0.0) return f;
  const double wavelen = 2.0 * 3.141592653589793 / f;
  if (wavelen < sc.orig / sc.high) return f;
  if (wavelen > sc.orig / sc.low) return f / sc.factor;
  const double m = (sc.orig / wavelen - sc.low) / (sc.high - sc.low);
  return (1.0 - m) * f / sc.factor + m * f;
}

__global__ void rope_kernel(uint16_t* __restrict__ x, int64_t T, int64_t ld, int n_heads, int head_dim, int seq,
                            double theta, RopeScale sc, int inverse) {
  int half = head_dim >> 1;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * half) return;
  int64_t row = idx / half;
  int i = (int)(idx - row * half);
  int pos = (int)(row % seq);
  double ang = (double)pos * rope_inv_freq(i, head_dim, theta, sc);
  double sd, cd;
  sincos(ang, &sd, &cd);
  float c = (float)cd, sn = inverse ? -(float)sd : (float)sd;
  uint16_t* xr = x + row * ld;
  for (int h = 0; h < n_heads; ++h) {
    uint16_t* p = xr + (int64_t)h * head_dim;
    float x1 = bf2f(p[i]), x2 = bf2f(p[i + half]);
    p[i] = f2bf(x1 * c - x2 * sn);
    p[i + half] = f2bf(x2 * c + x1 * sn);
  }
}

lsl_status rope_launch(uint16_t* x, int64_t T, int64_t ld, int n_heads, int head_dim, int seq, float theta,
                       const lsl_rope_scaling* scaling, int inverse, hipStream_t s) {
  if (T == 0) return LSL_OK;
  int64_t n = T * (head_dim / 2);
  RopeScale sc{0.0, 0.0, 0.0, 0.0};
  if (scaling && scaling->factor != 0.f)
    sc = RopeScale{scaling->factor, scaling->low_freq_factor, scaling->high_freq_factor,
                   scaling->original_max_position};
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, T, ld, n_heads, head_dim,
                     seq, (double)theta, sc, inverse);
  return check_launch("rope");
}

// ---------------------------------------------------------------- SwiGLU
LSL_DEV float sigm(float g) { return 1.0f / (1.0f + expf(-g)); }

__global__ void swiglu_fwd_kernel(const uint16_t* __restrict__ gu, int64_t T, int64_t I, uint16_t* __restrict__ a) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one per 8 outputs
  int64_t per = I / 8;
  if (idx >= T * per) return;
  int64_t t = idx / per, c = (idx - t * per) * 8;
  u32x4 g = *reinterpret_cast<const u32x4*>(gu + t * 2 * I + c);
  u32x4 u = *reinterpret_cast<const u32x4*>(gu + t * 2 * I + I + c);
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float g0 = lo_bf(g[j]), g1 = hi_bf(g[j]);
    o[j] = pack2(g0 * sigm(g0) * lo_bf(u[j]), g1 * sigm(g1) * hi_bf(u[j]));
  }
  *reinterpret_cast<u32x4*>(a + t * I + c) = o;
}

__global__ void swiglu_bwd_kernel(const uint16_t* __restrict__ gu, const uint16_t* __restrict__ da, int64_t T, int64_t I,
                                  uint16_t* __restrict__ dgu) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t per = I / 8;
  if (idx >= T * per) return;
  int64_t t = idx / per, c = (idx - t * per) * 8;
  u32x4 g = *reinterpret_cast<const u32x4*>(gu + t * 2 * I + c);
  u32x4 u = *reinterpret_cast<const u32x4*>(gu + t * 2 * I + I + c);
  u32x4 d = *reinterpret_cast<const u32x4*>(da + t * I + c);
  u32x4 og, ou;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float gg[2] = {lo_bf(g[j]), hi_bf(g[j])}, uu[2] = {lo_bf(u[j]), hi_bf(u[j])}, dd[2] = {lo_bf(d[j]), hi_bf(d[j])};
    float rg[2], ru[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float sg = sigm(gg[e]);
      rg[e] = dd[e] * uu[e] * sg * (1.0f + gg[e] * (1.0f - sg));
      ru[e] = dd[e] * gg[e] * sg;
    }
    og[j] = pack2(rg[0], rg[1]);
    ou[j] = pack2(ru[0], ru[1]);
  }
  *reinterpret_cast<u32x4*>(dgu + t * 2 * I + c) = og;
  *reinterpret_cast<u32x4*>(dgu + t * 2 * I + I + c) = ou;
}

lsl_status swiglu_fwd_launch(const uint16_t* gu, int64_t T, int64_t I, uint16_t* a, hipStream_t s) {
  if (T == 0) return LSL_OK;
  int64_t n = T * (I / 8);
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gu, T, I, a);
  return check_launch("swiglu_fwd");
}
lsl_status swiglu_bwd_launch(const uint16_t* gu, const uint16_t* da, int64_t T, int64_t I, uint16_t* dgu, hipStream_t s) {
  if (T == 0) return LSL_OK;
  int64_t n = T * (I / 8);
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gu, da, T, I, dgu);
  return check_launch("swiglu_bwd");
}

// ---------------------------------------------------------------- embedding
__global__ void embed_kernel(const uint16_t* __restrict__ table, const int32_t* __restrict__ ids, int64_t T, int64_t H,
                             int64_t V, uint16_t* __restrict__ out) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t per = H / 8;
  if (idx >= T * per) return;
  int64_t t = idx / per, c = (idx - t * per) * 8;
  int64_t id = ids[t];
  u32x4 v = (id >= 0 && id < V) ? *reinterpret_cast<const u32x4*>(table + id * H + c) : u32x4{0, 0, 0, 0};
  *reinterpret_cast<u32x4*>(out + t * H + c) = v;
}

// ---------------------------------------------------------------- AdamW
__global__ void adamw_kernel(float* __restrict__ p, uint16_t* __restrict__ pb, const float* __restrict__ g,
                             float* __restrict__ m, float* __restrict__ v, int64_t n, float lr, float b1, float b2,
                             float eps, float decay, float bc1, float bc2) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float gi = g[i];
  float pi = p[i] * decay;
  float mi = b1 * m[i] + (1.0f - b1) * gi;
  float vi = b2 * v[i] + (1.0f - b2) * gi * gi;
  pi -= lr * (mi / bc1) / (sqrtf(vi / bc2) + eps);
  p[i] = pi; m[i] = mi; v[i] = vi;
  if (pb) pb[i] = f2bf(pi);
}

}  // namespace lsl

using namespace lsl;

extern "C" lsl_status lsl_embed_fwd(const uint16_t* table, const int32_t* ids, int64_t T, int64_t H, int64_t V,
                                    uint16_t* out, lsl_stream stream) {
  if (T < 0 || H <= 0 || V <= 0 || H % 8)
    return set_error(LSL_ERR_INVALID_ARG, "lsl_embed_fwd: bad sizes (H must be a multiple of 8)");
  if (T == 0) return LSL_OK;
  if (!table || !ids || !out || !aligned(table, 16) || !aligned(out, 16) || !aligned(ids, 4))
    return set_error(LSL_ERR_INVALID_ARG, "lsl_embed_fwd: null or misaligned pointer");
  int64_t n = T * (H / 8);
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, table, ids, T,
                     H, V, out);
  return check_launch("embed");
}

extern "C" lsl_status lsl_adamw_step(float* p, uint16_t* p_bf16, const float* g, float* m, float* v, int64_t n,
                                     int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                                     lsl_stream stream) {
  if (n < 0 || step < 1) return set_error(LSL_ERR_INVALID_ARG, "lsl_adamw_step: n >= 0 and step >= 1 required");
  if (n == 0) return LSL_OK;
  if (!p || !g || !m || !v) return set_error(LSL_ERR_INVALID_ARG, "lsl_adamw_step: null pointer");
  float bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  float bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  float decay = 1.0f - lr * weight_decay;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, p, p_bf16, g,
                     m, v, n, lr, beta1, beta2, eps, decay, bc1, bc2);
  return check_launch("adamw");
}
