// HBM-bound steps of the decoder layer: RMSNorm forward/backward, rotary
// embedding, SwiGLU forward/backward, embedding gather and AdamW. One wave per
// row for the row reductions (wave64 shuffles, no LDS), 16-byte accesses.
#include "common.h"
#include "small.h"
#include <cmath>

namespace lsl {

// ---------------------------------------------------------------- RMSNorm
// One wave per row. The forward holds the lane's 16-byte chunks of the row
// (chunk c of lane L covers columns 8 (L + 64 c) .. + 7) in registers, so the
// row is read from HBM once and all of its loads are in flight together (rows
// up to 512 RMS_CHUNKS columns).
constexpr int RMS_CHUNKS = 16;

// y = bf16(x * r * w), r = 1 / sqrt(mean(x^2) + eps)
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                          int64_t T, int64_t H, float eps, uint16_t* __restrict__ y) {
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= T) return;
  const uint16_t* xr = x + row * H;
  u32x4 v[RMS_CHUNKS];
#pragma unroll
  for (int c = 0; c < RMS_CHUNKS; ++c) {
    const int64_t col = (int64_t)(lane + 64 * c) * 8;
    if (col < H) v[c] = *reinterpret_cast<const u32x4*>(xr + col);
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < RMS_CHUNKS; ++c)
    if ((int64_t)(lane + 64 * c) * 8 < H)
#pragma unroll
      for (int j = 0; j < 4; ++j) { float a = lo_bf(v[c][j]), b = hi_bf(v[c][j]); ss += a * a + b * b; }
  ss = wave_sum(ss);
  float r = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int c = 0; c < RMS_CHUNKS; ++c) {
    const int64_t col = (int64_t)(lane + 64 * c) * 8;
    if (col >= H) continue;
    u32x4 g = *reinterpret_cast<const u32x4*>(w + col);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack2(lo_bf(v[c][j]) * r * lo_bf(g[j]), hi_bf(v[c][j]) * r * hi_bf(g[j]));
    *reinterpret_cast<u32x4*>(y + row * H + col) = o;
  }
}

// dx = bf16(dres + r (w dy - x r^2 sum(x w dy) / H)). Two passes over the row
// (the second from L2): holding x and dy in registers would halve occupancy.
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
  if (H > 512 * RMS_CHUNKS) return set_error(LSL_ERR_UNSUPPORTED, "rmsnorm: hidden %lld > %d", (long long)H, 512 * RMS_CHUNKS);
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
// The inverse frequencies theta^(-2i/d) (optionally rescaled the Llama-3.1 way)
// are computed on the host in float64 and passed by value. A workgroup takes
// ROPE_ROWS rows: first the float64 angle and its sine/cosine for each
// (row, i) into LDS, then every head's pairs (i, i + d/2) of those rows are
// rotated in float32 four at a time (8-byte accesses) and rounded to bf16 in
// place.
struct RopeFreq {
  double inv[64];  // head_dim / 2 <= 64
};

static RopeFreq rope_freq(int head_dim, double theta, const lsl_rope_scaling* sc) {
  RopeFreq fr{};
  const double pi = 3.141592653589793;
  for (int i = 0; i < head_dim / 2; ++i) {
    double f = std::pow(theta, -2.0 * (double)i / (double)head_dim);
    if (sc && sc->factor != 0.f) {
      const double factor = sc->factor, low = sc->low_freq_factor, high = sc->high_freq_factor;
      const double orig = sc->original_max_position;
      const double wavelen = 2.0 * pi / f;
      if (wavelen > orig / low) {
        f = f / factor;
      } else if (wavelen >= orig / high) {
        const double m = (orig / wavelen - low) / (high - low);
        f = (1.0 - m) * f / factor + m * f;
      }
    }
    fr.inv[i] = f;
  }
  return fr;
}

constexpr int ROPE_ROWS = 4;

__global__ __launch_bounds__(256) void rope_kernel(uint16_t* __restrict__ x, int64_t T, int64_t ld, int n_heads,
                                                   int head_dim, int seq, RopeFreq fr, int inverse) {
  __shared__ float cs[ROPE_ROWS][64], sn[ROPE_ROWS][64];
  const int half = head_dim >> 1;
  const int64_t r0 = (int64_t)blockIdx.x * ROPE_ROWS;
  for (int t = threadIdx.x; t < ROPE_ROWS * half; t += blockDim.x) {
    const int rr = t / half, i = t - rr * half;
    const int64_t row = r0 + rr;
    if (row >= T) continue;
    const double ang = (double)(row % seq) * fr.inv[i];
    double sd, cd;
    sincos(ang, &sd, &cd);
    cs[rr][i] = (float)cd;
    sn[rr][i] = inverse ? -(float)sd : (float)sd;
  }
  __syncthreads();
  const int q4 = half >> 2;          // groups of 4 pairs per head
  const int per_row = n_heads * q4;
  for (int t = threadIdx.x; t < ROPE_ROWS * per_row; t += blockDim.x) {
    const int rr = t / per_row, rem = t - rr * per_row;
    const int h = rem / q4, g = rem - h * q4;
    const int64_t row = r0 + rr;
    if (row >= T) continue;
    uint16_t* p = x + row * ld + (int64_t)h * head_dim + 4 * g;
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + half);
    float x1[4] = {lo_bf(a[0]), hi_bf(a[0]), lo_bf(a[1]), hi_bf(a[1])};
    float x2[4] = {lo_bf(b[0]), hi_bf(b[0]), lo_bf(b[1]), hi_bf(b[1])};
    float o1[4], o2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = cs[rr][4 * g + e], s = sn[rr][4 * g + e];
      o1[e] = x1[e] * c - x2[e] * s;
      o2[e] = x2[e] * c + x1[e] * s;
    }
    *reinterpret_cast<u32x2*>(p) = u32x2{pack2(o1[0], o1[1]), pack2(o1[2], o1[3])};
    *reinterpret_cast<u32x2*>(p + half) = u32x2{pack2(o2[0], o2[1]), pack2(o2[2], o2[3])};
  }
}

lsl_status rope_launch(uint16_t* x, int64_t T, int64_t ld, int n_heads, int head_dim, int seq, float theta,
                       const lsl_rope_scaling* scaling, int inverse, hipStream_t s) {
  if (head_dim % 8 || head_dim > 128)
    return set_error(LSL_ERR_UNSUPPORTED, "rope: head_dim %d (a multiple of 8, at most 128)", head_dim);
  if (T == 0) return LSL_OK;
  const RopeFreq fr = rope_freq(head_dim, (double)theta, scaling);
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((T + ROPE_ROWS - 1) / ROPE_ROWS)), dim3(256), 0, s, x, T, ld,
                     n_heads, head_dim, seq, fr, inverse);
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
